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



def test_noalloc_forward_replays_in_a_graph(gpu):
    """The no-allocation forward captured in a HIP graph (torch.cuda.CUDAGraph,
    the use it exists for) and replayed four times, with eager library calls and
    synchronisations between the replays and new inputs copied into the captured
    buffers before two of them: every replay equals the eager flce_forward (with
    a workspace) of the same inputs, bit for bit."""
    lib = gpu.load()
    N, H, V, dtype, red = 1000, 512, 5000, "bf16", 0
    dt = DT[dtype]
    note(f"[no-alloc graph] N={N} H={H} V={V} {dtype}")
    x, W, t = make_inputs(N, H, V, dtype, seed=61)
    xd, Wd, td = to_dev(x, dtype), to_dev(W, dtype), torch.from_numpy(t).cuda()
    loss = torch.zeros(1, device="cuda")
    lse = torch.zeros(N, device="cuda")
    zt = torch.zeros(N, device="cuda")
    ws = torch.empty(lib.flce_forward_workspace_bytes(N, H, V, dt), dtype=torch.uint8, device="cuda")

    def noalloc(stream):
        return lib.flce_forward_noalloc(xd.data_ptr(), Wd.data_ptr(), td.data_ptr(), N, H, V, dt, red,
                                        loss.data_ptr(), lse.data_ptr(), zt.data_ptr(), stream)

    def eager_reference():
        rl = torch.full((1,), float("nan"), device="cuda")
        rs = torch.full((N,), float("nan"), device="cuda")
        rz = torch.full((N,), float("nan"), device="cuda")
        code = lib.flce_forward(xd.data_ptr(), Wd.data_ptr(), td.data_ptr(), N, H, V, dt, red, rl.data_ptr(),
                                rs.data_ptr(), rz.data_ptr(), ws.data_ptr(), ws.numel(),
                                torch.cuda.current_stream().cuda_stream)
        assert code == 0, lib.flce_status_string(code)
        torch.cuda.synchronize()
        return rl.cpu(), rs.cpu(), rz.cpu()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # eager first call: looks the scratch address up
        assert noalloc(side.cuda_stream) == 0
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        code = noalloc(torch.cuda.current_stream().cuda_stream)
    assert code == 0, lib.flce_status_string(code)
    torch.cuda.synchronize()
    for rep in range(4):
        if rep in (1, 3):  # new inputs in the captured buffers
            x2, W2, t2 = make_inputs(N, H, V, dtype, seed=61 + rep)
            xd.copy_(to_dev(x2, dtype))
            Wd.copy_(to_dev(W2, dtype))
            td.copy_(torch.from_numpy(t2).cuda())
        loss.fill_(float("nan"))
        lse.fill_(float("nan"))
        zt.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (loss.cpu(), lse.cpu(), zt.cpu())
        ref = eager_reference()
        assert all(torch.isfinite(g).all() for g in got), rep
        assert all(torch.equal(g, r) for g, r in zip(got, ref)), rep
