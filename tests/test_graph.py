"""The backward, the forward and the single-call forward + backward captured in
HIP graphs (torch.cuda.CUDAGraph) and replayed.

The shape has balanced gradient launches (grad_W: 9 hidden x 32 vocabulary tiles =
288 on 256 workgroups), so the replays also run the flag-clearing kernel and the
partial-sum hand-over between workgroups; the dlogit launch (3 x 32 tiles, K =
2304) runs as K pieces.  Every replay must equal an eager backward of the same
inputs bit for bit."""
import pytest
import torch

from lm_head_linear_tiled_amd.inputs import make_inputs
from tests.gpu_util import note, to_dev


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_replays_in_a_graph(gpu, dtype):
    """Capture flce_backward once, then replay it four times with eager library
    calls and synchronisations between the replays and new inputs (x, W, targets
    and the matching lse) copied into the captured buffers before replays 1 and 3:
    grad_x and grad_W of every replay equal the eager backward's, bit for bit."""
    N, H, V, red = 600, 2304, 8000, "sum"
    note(f"[graph backward] N={N} H={H} V={V} {dtype}")
    x, W, t = make_inputs(N, H, V, dtype, seed=81)
    xd, Wd, td = to_dev(x, dtype), to_dev(W, dtype), torch.from_numpy(t).cuda()
    gl = torch.tensor([0.9], device="cuda")
    _, lse = gpu.flce_forward(xd, Wd, td, red)
    bits = torch.int16 if dtype == "bf16" else torch.int32

    def eager():
        gx, gW = gpu.flce_backward(xd, Wd, td, lse, gl, red)
        torch.cuda.synchronize()
        return gx.view(bits).clone(), gW.view(bits).clone()

    ref = eager()
    # warm-up on a side stream (the library's first call per device, torch's caches)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gpu.flce_backward(xd, Wd, td, lse, gl, red)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cgx, cgW = gpu.flce_backward(xd, Wd, td, lse, gl, red)
    torch.cuda.synchronize()
    for rep in range(4):
        if rep in (1, 3):  # new inputs in the captured buffers
            x2, W2, t2 = make_inputs(N, H, V, dtype, seed=81 + rep)
            xd.copy_(to_dev(x2, dtype))
            Wd.copy_(to_dev(W2, dtype))
            td.copy_(torch.from_numpy(t2).cuda())
            _, lse2 = gpu.flce_forward(xd, Wd, td, red)
            lse.copy_(lse2)
            torch.cuda.synchronize()
            ref = eager()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(cgx.view(bits), ref[0]), f"replay {rep}: grad_x"
        assert torch.equal(cgW.view(bits), ref[1]), f"replay {rep}: grad_W"
        # eager work between the replays
        assert torch.equal(eager()[1], ref[1])


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward_and_single_call_replay_in_graphs(gpu, dtype):
    """flce_forward and flce_forward_backward (no grad_loss: the implicit 1 is
    written by a kernel) each captured once and replayed four times, new inputs
    copied into the captured buffers before replays 1 and 3, eager library calls
    and synchronisations between the replays: loss, lse and both gradients of
    every replay equal an eager call's, bit for bit."""
    N, H, V, red = 600, 2304, 8000, "mean"
    note(f"[graph forward, forward+backward] N={N} H={H} V={V} {dtype}")
    x, W, t = make_inputs(N, H, V, dtype, seed=91)
    xd, Wd, td = to_dev(x, dtype), to_dev(W, dtype), torch.from_numpy(t).cuda()
    bits = torch.int16 if dtype == "bf16" else torch.int32

    def eager():
        loss, lse = gpu.flce_forward(xd, Wd, td, red)
        l2, lse2, gx, gW = gpu.flce_forward_backward(xd, Wd, td, red)
        torch.cuda.synchronize()
        return [a.clone() for a in (loss, lse, l2, lse2)] + [gx.view(bits).clone(), gW.view(bits).clone()]

    ref = eager()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gpu.flce_forward(xd, Wd, td, red)
        gpu.flce_forward_backward(xd, Wd, td, red)
    torch.cuda.synchronize()
    g_fwd, g_fb = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_fwd):
        c_loss, c_lse = gpu.flce_forward(xd, Wd, td, red)
    with torch.cuda.graph(g_fb):
        c_l2, c_lse2, c_gx, c_gW = gpu.flce_forward_backward(xd, Wd, td, red)
    torch.cuda.synchronize()
    for rep in range(4):
        if rep in (1, 3):  # new inputs in the captured buffers
            x2, W2, t2 = make_inputs(N, H, V, dtype, seed=91 + rep)
            xd.copy_(to_dev(x2, dtype))
            Wd.copy_(to_dev(W2, dtype))
            td.copy_(torch.from_numpy(t2).cuda())
            torch.cuda.synchronize()
            ref = eager()
        g_fwd.replay()
        g_fb.replay()
        torch.cuda.synchronize()
        got = [c_loss, c_lse, c_l2, c_lse2, c_gx.view(bits), c_gW.view(bits)]
        for name, a, b in zip(("loss", "lse", "fb loss", "fb lse", "grad_x", "grad_W"), got, ref):
            assert torch.equal(a, b), f"replay {rep}: {name}"
        # eager work between the replays
        assert torch.equal(eager()[5], ref[5])
