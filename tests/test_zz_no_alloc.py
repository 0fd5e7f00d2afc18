"""flce_forward_noalloc (the forward for callers that cannot allocate: its
workspace is the library's static device scratch) against flce_forward with a
workspace, through the C ABI: bit-identical loss, lse and target logits on two
calls in a row, the second with a smaller input (the scratch keeps the first
call's contents, which must not matter)."""
import ctypes

import numpy as np
import pytest
import torch

from lm_head_linear_tiled_amd.inputs import make_inputs
from tests.gpu_util import note, to_dev

pytestmark = pytest.mark.gpu

DT = {"f32": 0, "bf16": 1}


def _call(lib, N, H, V, dtype, red, seed):
    x, W, t = make_inputs(N, H, V, dtype, seed=seed)
    xd, Wd, td = to_dev(x, dtype), to_dev(W, dtype), torch.from_numpy(t).cuda()
    s = torch.cuda.current_stream().cuda_stream
    dt = DT[dtype]
    outs = []
    for noalloc in (False, True):
        loss = torch.full((1,), float("nan"), device="cuda")
        lse = torch.full((N,), float("nan"), device="cuda")
        zt = torch.full((N,), float("nan"), device="cuda")
        if noalloc:
            code = lib.flce_forward_noalloc(xd.data_ptr(), Wd.data_ptr(), td.data_ptr(), N, H, V, dt, red,
                                            loss.data_ptr(), lse.data_ptr(), zt.data_ptr(), s)
        else:
            ws = torch.empty(lib.flce_forward_workspace_bytes(N, H, V, dt), dtype=torch.uint8, device="cuda")
            code = lib.flce_forward(xd.data_ptr(), Wd.data_ptr(), td.data_ptr(), N, H, V, dt, red,
                                    loss.data_ptr(), lse.data_ptr(), zt.data_ptr(), ws.data_ptr(), ws.numel(), s)
        assert code == 0, lib.flce_status_string(code)
        torch.cuda.synchronize()
        outs.append((loss.cpu(), lse.cpu(), zt.cpu()))
    (l0, s0, z0), (l1, s1, z1) = outs
    assert torch.isfinite(l0).all() and torch.isfinite(s0).all() and torch.isfinite(z0).all()
    assert torch.equal(l0, l1) and torch.equal(s0, s1) and torch.equal(z0, z1)


def test_noalloc_forward_matches_workspace_forward(gpu):
    lib = gpu.load()
    # first a large call (many token tiles and vocabulary splits fill much of the
    # scratch), then a smaller one of the other type over the stale contents
    note("[no-alloc] N=5000 H=512 V=20000 bf16, then N=300 H=256 V=1000 f32")
    _call(lib, 5000, 512, 20000, "bf16", 0, seed=51)
    _call(lib, 300, 256, 1000, "f32", 1, seed=52)

