"""Out-of-bounds guards: inputs sit inside NaN-poisoned allocations and outputs
between NaN canary bands; any read or write past N, V or H shows up."""
import numpy as np
import pytest
import torch

from lm_head_linear_tiled_amd import binding as B
from lm_head_linear_tiled_amd.inputs import make_inputs
from tests.gpu_util import note, to_dev

pytestmark = pytest.mark.gpu

GUARD = 64  # rows of poison before and after every buffer


def poisoned_like(t):
    """A copy of t placed GUARD rows into a NaN-filled buffer; returns (view, whole)."""
    rows, cols = t.shape if t.dim() == 2 else (t.shape[0], 1)
    whole = torch.full((rows + 2 * GUARD, cols), float("nan"), dtype=t.dtype, device=t.device)
    view = whole[GUARD:GUARD + rows]
    view.copy_(t.reshape(rows, cols))
    return (view if t.dim() == 2 else view.reshape(rows)), whole


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_poisoned_inputs_and_canaries(gpu, dtype):
    N, H, V = 1269, 1000 if dtype == "f32" else 1000, 10000
    note(f"[oob] {dtype} N={N} H={H} V={V}")
    x, W, t = make_inputs(N, H, V, dtype, seed=21)
    xd, Wd, td = to_dev(x, dtype), to_dev(W, dtype), torch.from_numpy(t).cuda()
    ref_loss, ref_lse = gpu.flce_forward(xd, Wd, td, "sum")
    ref_gx, ref_gW = gpu.flce_backward(xd, Wd, td, ref_lse, torch.ones(1, device="cuda"), "sum")

    xp, _ = poisoned_like(xd)
    Wp, _ = poisoned_like(Wd)
    lib = gpu.load()
    dt = 0 if dtype == "f32" else 1
    loss = torch.full((3,), float("nan"), device="cuda")
    lse_v, lse_w = poisoned_like(torch.zeros(N, device="cuda"))
    gx_v, gx_w = poisoned_like(torch.zeros(N, H, dtype=xd.dtype, device="cuda"))
    gW_v, gW_w = poisoned_like(torch.zeros(V, H, dtype=xd.dtype, device="cuda"))
    fws = torch.empty(lib.flce_forward_workspace_bytes(N, H, V, dt), dtype=torch.uint8, device="cuda")
    bws = torch.empty(lib.flce_backward_workspace_bytes(N, H, V, dt), dtype=torch.uint8, device="cuda")
    bws.fill_(0xFF)  # NaN bit patterns in the workspace must never leak either
    gl = torch.ones(1, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert lib.flce_forward(xp.data_ptr(), Wp.data_ptr(), td.data_ptr(), N, H, V, dt, 1, loss[1:].data_ptr(),
                            lse_v.data_ptr(), None, fws.data_ptr(), fws.numel(), s) == 0
    assert lib.flce_backward(xp.data_ptr(), Wp.data_ptr(), td.data_ptr(), lse_v.data_ptr(), gl.data_ptr(), N, H, V,
                             dt, 1, gx_v.data_ptr(), gW_v.data_ptr(), bws.data_ptr(), bws.numel(), s) == 0
    torch.cuda.synchronize()
    assert torch.isnan(loss[0]) and torch.isnan(loss[2]) and loss[1] == ref_loss[0]
    for whole, view, ref in ((lse_w, lse_v, ref_lse), (gx_w, gx_v, ref_gx), (gW_w, gW_v, ref_gW)):
        assert torch.equal(view.reshape(ref.shape), ref)
        assert torch.isnan(whole[:GUARD].float()).all() and torch.isnan(whole[-GUARD:].float()).all()
