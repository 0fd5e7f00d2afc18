"""HIP path against the CPU oracle, element by element, on seeded inputs."""
import math

import numpy as np
import pytest
import torch

import oracle
from lm_head_linear_tiled_amd.inputs import WORKLOADS, make_inputs, widen
from tests.gpu_util import assert_parity, note, run_hip, to_dev, to_f64

pytestmark = pytest.mark.gpu


def oracle_all(x, W, t, dtype, reduction, grad_loss=1.0):
    xf, Wf = widen(x, dtype), widen(W, dtype)
    loss, lse, zt = oracle.forward(xf, Wf, t, reduction)
    gx, gW = oracle.backward(xf, Wf, t, reduction, grad_loss)
    return loss, lse, zt, gx, gW


def contractions(timer):
    """The kernel sequence of a timed call."""
    return [k for k, _ in timer.durations()]


def check_case(gpu, N, H, V, dtype, reduction, seed=0, grad_loss=1.0, t=None, bwd_ws_bytes=None, **kw):
    note(f"[parity] N={N} H={H} V={V} {dtype} {reduction} seed={seed} ws={bwd_ws_bytes}")
    x, W, t0 = make_inputs(N, H, V, dtype, seed=seed, **kw)
    t = t0 if t is None else np.asarray(t, dtype=np.int64)
    got = run_hip(gpu, x, W, t, dtype, reduction, grad_loss, bwd_ws_bytes)
    assert_parity(got, *oracle_all(x, W, t, dtype, reduction, grad_loss), dtype)
    return got


@pytest.mark.parametrize("name,reduction", [
    ("tiny", "mean"), ("ragged", "sum"), ("ragged", "mean"), ("llama2_bf16", "mean"), ("llama2_f32", "mean"),
])
def test_workload_parity(gpu, name, reduction):
    w = WORKLOADS[name]
    check_case(gpu, w.N, w.H, w.V, w.dtype, reduction)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_multi_tile_ragged(gpu, dtype, reduction):
    check_case(gpu, 300, 264, 1000, dtype, reduction, seed=3, grad_loss=0.7)


@pytest.mark.parametrize("N,H,V,dtype", [
    (1, 4, 1, "f32"), (1, 8, 2, "bf16"), (2, 8, 3, "f32"), (129, 64, 129, "bf16"), (127, 36, 257, "f32"),
    (257, 16, 130, "bf16"),
])
def test_edge_shapes(gpu, N, H, V, dtype):
    check_case(gpu, N, H, V, dtype, "sum", seed=N + V)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_targets_at_tile_edges(gpu, dtype):
    N, H, V = 256, 128, 1000
    t = np.array([0, V - 1, 127, 128, 255, 256, 895, 896] * (N // 8), dtype=np.int64)
    check_case(gpu, N, H, V, dtype, "mean", seed=5, t=t)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_all_targets_equal(gpu, dtype):
    """Every token has the same target: the heaviest single-row update of grad_W."""
    N, H, V = 512, 128, 3000
    check_case(gpu, N, H, V, dtype, "sum", seed=6, t=np.full(N, 1234))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_small_workspace_panels(gpu, dtype, reduction):
    """The minimum workspace forces many dlogit panels and token chunks, so every
    accumulation path (first, middle, last panel and chunk) runs."""
    N, H, V = 700, 96, 1500
    nmin = gpu.backward_min_workspace_bytes(N, H, V, torch.float32 if dtype == "f32" else torch.bfloat16)
    check_case(gpu, N, H, V, dtype, reduction, seed=7, grad_loss=1.5, bwd_ws_bytes=nmin)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_grad_x_split_k(gpu, dtype, reduction):
    """Few grad_x output tiles (2 x 2): the panel's vocabulary is split over four
    workgroups per tile, the last range ragged, and bwd_gx_reduce adds them."""
    N, H, V = 512, 512, 9000
    got = check_case(gpu, N, H, V, dtype, reduction, seed=21, grad_loss=0.9)
    x, W, t = make_inputs(N, H, V, dtype, seed=21)
    xd, Wd, td = to_dev(x, dtype), to_dev(W, dtype), torch.from_numpy(t).cuda()
    bt = gpu.KernelTimer(16)
    gpu.flce_backward(xd, Wd, td, got["raw"]["lse"], torch.tensor([0.9], device="cuda"), reduction, timer=bt)
    torch.cuda.synchronize()
    assert contractions(bt) == ["bwd_dlogits", "bwd_grad_w", "bwd_grad_x", "bwd_gx_reduce"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_grad_x_split_k_several_panels(gpu, dtype):
    """Split grad_x launches over three vocabulary panels: the first split of each
    tile starts from the earlier panels' partial sums."""
    N, H, V = 512, 256, 40000
    nws = gpu.backward_workspace_bytes(N, H, V, torch.float32 if dtype == "f32" else torch.bfloat16) // 2
    check_case(gpu, N, H, V, dtype, "mean", seed=22, bwd_ws_bytes=nws)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_whole_slice_copies_with_ragged_rows(gpu, dtype):
    """Tokens a multiple of the K slice but not of the tile (N = 320, H = 256): the
    forward and dlogits copy x and W by whole K slices with rows past N and V left
    to the buffer range check, and grad_W runs its whole-slice loop over K = 320."""
    check_case(gpu, 320, 256, 3000, dtype, "sum", seed=24, grad_loss=1.25)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_grad_x_sums_over_wide_panels(gpu, dtype):
    """grad_x over two vocabulary panels of many K slices each, split in K: later
    panels start from the earlier panels' float32 sums; ragged tokens and hidden
    size (H = 320: the second hidden tile is mostly past H)."""
    N, H, V = 300, 320, 12000
    nws = gpu.backward_workspace_bytes(N, H, V, torch.float32 if dtype == "f32" else torch.bfloat16) // 2
    check_case(gpu, N, H, V, dtype, "sum", seed=23, grad_loss=0.7, bwd_ws_bytes=nws)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_grad_x_over_panel_pairs(gpu, dtype):
    """All tokens in one chunk and several vocabulary panels (the default
    workspace): two panels are kept at once, each in its own block, and grad_x runs
    once per pair with its copies crossing from the first block to the second; the
    odd, ragged last panel forms a group of its own.  One grad_x output tile, so
    each group's vocabulary is split in K and the ranges cross the block boundary."""
    N, H, V = 200, 72, 600000
    got = check_case(gpu, N, H, V, dtype, "mean", seed=25, grad_loss=1.1)
    x, W, t = make_inputs(N, H, V, dtype, seed=25)
    xd, Wd, td = to_dev(x, dtype), to_dev(W, dtype), torch.from_numpy(t).cuda()
    bt = gpu.KernelTimer(64)
    gpu.flce_backward(xd, Wd, td, got["raw"]["lse"], torch.tensor([1.1], device="cuda"), "mean", timer=bt)
    torch.cuda.synchronize()
    panels = 3 if dtype == "bf16" else 5  # 128 MB panels of 256 (padded) tokens: 262144 / 131072 entries
    seq = []
    for p in range(panels):
        seq += ["bwd_dlogits", "bwd_grad_w"]
        if p % 2 == 1 or p == panels - 1:
            seq += ["bwd_grad_x", "bwd_gx_reduce"]
    # (a ragged last panel's grad_W launch may also be followed by its split tail)
    assert [k for k in contractions(bt) if k not in ("tail_pieces", "tail_fixup")] == seq


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_w_zero_closed_form(gpu, dtype):
    """W = 0: lse = ln V and loss = ln V (mean), grad_x = 0 exactly."""
    N, H, V = 200, 64, 777
    x, W, t = make_inputs(N, H, V, dtype, seed=8)
    W = np.zeros_like(W)
    got = run_hip(gpu, x, W, t, dtype, "mean")
    assert abs(got["loss"] - math.log(V)) <= 2e-6 * math.log(V)
    np.testing.assert_allclose(got["lse"], math.log(V), rtol=2e-6)
    assert np.all(got["gx"] == 0.0)
    xf = widen(x, dtype)
    want = np.tile(xf.sum(axis=0) / V / N, (V, 1))
    for i in range(N):
        want[t[i]] -= xf[i] / N
    tol = 1e-6 if dtype == "f32" else 1e-2 * np.abs(want).max()
    assert np.abs(got["gW"] - want).max() <= tol


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_integer_inputs_gather_exact(gpu, dtype):
    """Integer-valued x and W make every logit exact in fp32 whatever the
    summation order, so the gathered target logit must equal the oracle's bit
    for bit and lse must agree to a few fp32 ulps."""
    N, H, V = 300, 256, 2000
    g = np.random.Generator(np.random.PCG64(9))
    xi = g.integers(-8, 9, size=(N, H)).astype(np.float32)
    Wi = g.integers(-8, 9, size=(V, H)).astype(np.float32) / 64.0  # still exact in bf16 (k / 64)
    t = g.integers(0, V, size=N)
    if dtype == "bf16":
        from lm_head_linear_tiled_amd.inputs import bf16_bits_from_f32
        x, W = bf16_bits_from_f32(xi), bf16_bits_from_f32(Wi)
    else:
        x, W = xi, Wi
    got = run_hip(gpu, x, W, t, dtype, "mean")
    _, lse, zt = oracle.forward(widen(x, dtype), widen(W, dtype), t, "mean")
    assert np.array_equal(got["zt"], zt), "target logit not bit-exact"
    ulp = np.spacing(np.abs(lse).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got["lse"] - lse) <= 4 * ulp + 1e-6)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_extreme_logits_finite(gpu, dtype):
    """Logits of magnitude ~1e3 stay finite and match the oracle to the rounding
    bound of fp32 logits.  A dot product of length H accumulated in fp32 errs by at
    most delta = (H + 2) u sum_h |x_h||W_vh| (u = 2^-24); softmax and lse inherit an
    absolute error <= 2 delta, so each loss term errs by <= 3 delta and every
    gradient, normalised by max|grad|, by <= 2 delta on top of the usual bar."""
    N, H, V = 100, 64, 500
    note(f"[parity] extreme logits {dtype}")
    x, W, t = make_inputs(N, H, V, dtype, seed=10, w_std=40.0)
    got = run_hip(gpu, x, W, t, dtype, "sum")
    loss, lse, zt, gx, gW = oracle_all(x, W, t, dtype, "sum")
    xf, Wf = widen(x, dtype), widen(W, dtype)
    assert np.abs(xf @ Wf.T).max() > 500
    delta = (H + 2) * 2.0 ** -24 * (np.abs(xf) @ np.abs(Wf).T).max()
    for k in ("gx", "gW", "lse", "zt"):
        assert np.all(np.isfinite(got[k])), k
    assert abs(got["loss"] - loss) <= 3 * delta * N + 1e-5 * abs(loss)
    assert np.abs(got["lse"] - lse).max() <= 2 * delta + 1e-5 * np.abs(lse).max()
    base = 1e-4 if dtype == "f32" else 1e-2
    for g, r in ((got["gx"], gx), (got["gW"], gW)):
        assert np.abs(g - r).max() / np.abs(r).max() <= base + 2 * delta


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_deterministic(gpu, dtype):
    """Forward and backward are bitwise reproducible (no atomics, fixed order)."""
    N, H, V = 513, 128, 4099
    x, W, t = make_inputs(N, H, V, dtype, seed=11)
    a = run_hip(gpu, x, W, t, dtype, "mean")
    b = run_hip(gpu, x, W, t, dtype, "mean")
    for k in ("lse", "zt", "gx", "gW"):
        assert np.array_equal(a[k], b[k]), k
    assert a["loss"] == b["loss"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_grad_loss_linear(gpu, dtype):
    """Edge tiles only (N = 130 < one token tile): there D = s (p - onehot) is formed
    in fp32 and then rounded, and a power-of-two scale commutes with every rounding.
    (Interior tiles fold s into the exponent; test_negative_and_zero_grad_loss.)"""
    N, H, V = 130, 64, 300
    x, W, t = make_inputs(N, H, V, dtype, seed=12)
    a = run_hip(gpu, x, W, t, dtype, "sum", grad_loss=1.0)
    b = run_hip(gpu, x, W, t, dtype, "sum", grad_loss=-0.25)
    assert np.array_equal(b["gx"], -0.25 * a["gx"]) and np.array_equal(b["gW"], -0.25 * a["gW"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("grad_loss", [-0.6, 0.0])
def test_negative_and_zero_grad_loss(gpu, dtype, grad_loss):
    """Every tile inside N and V: the dlogit scale enters the exponent as
    log2|grad_loss| and its sign as a sign flip, the one-hot term is patched in
    afterwards; a zero upstream gradient gives exactly zero gradients."""
    N, H, V = 512, 256, 1024
    got = check_case(gpu, N, H, V, dtype, "mean", seed=31, grad_loss=grad_loss)
    if grad_loss == 0.0:
        assert not np.any(got["gx"]) and not np.any(got["gW"])


def test_autograd_matches_direct(gpu):
    N, H, V = 200, 128, 999
    x, W, t = make_inputs(N, H, V, "bf16", seed=13)
    xd = to_dev(x, "bf16").requires_grad_(True)
    Wd = to_dev(W, "bf16").requires_grad_(True)
    td = torch.from_numpy(t).cuda()
    loss = gpu.flce_loss(xd, Wd, td, "mean")
    (2.0 * loss).backward()
    got = run_hip(gpu, x, W, t, "bf16", "mean", grad_loss=2.0)
    assert loss.item() == got["loss"]
    assert np.array_equal(to_f64(xd.grad), got["gx"]) and np.array_equal(to_f64(Wd.grad), got["gW"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("with_grad_loss", [False, True])
def test_forward_backward_single_call(gpu, dtype, with_grad_loss):
    """One call gives the same bits as flce_forward then flce_backward."""
    N, H, V = 700, 96, 1500
    note(f"[parity] single call {dtype} grad_loss={with_grad_loss}")
    x, W, t = make_inputs(N, H, V, dtype, seed=14)
    xd, Wd, td = to_dev(x, dtype), to_dev(W, dtype), torch.from_numpy(t).cuda()
    gl = torch.tensor([0.75 if with_grad_loss else 1.0], device="cuda")
    loss, lse, gx, gW = gpu.flce_forward_backward(xd, Wd, td, "sum", grad_loss=gl if with_grad_loss else None)
    l2, lse2 = gpu.flce_forward(xd, Wd, td, "sum")
    gx2, gW2 = gpu.flce_backward(xd, Wd, td, lse2, gl, "sum")
    torch.cuda.synchronize()
    assert torch.equal(loss, l2) and torch.equal(lse, lse2)
    assert torch.equal(gx, gx2) and torch.equal(gW, gW2)
    # and against the oracle
    ref = oracle_all(x, W, t, dtype, "sum", float(gl.item()))
    got = dict(loss=float(loss.item()), lse=to_f64(lse), zt=None, gx=to_f64(gx), gW=to_f64(gW))
    assert_parity(got, ref[0], None, None, ref[3], ref[4], dtype)


def test_timed_variants_record_every_kernel(gpu):
    """The *_timed calls give the same bits as the plain calls and one event per kernel."""
    N, H, V = 300, 128, 2000
    x, W, t = make_inputs(N, H, V, "bf16", seed=15)
    xd, Wd, td = to_dev(x, "bf16"), to_dev(W, "bf16"), torch.from_numpy(t).cuda()
    ft, bt = gpu.KernelTimer(8), gpu.KernelTimer(64)
    l1, lse1 = gpu.flce_forward(xd, Wd, td, "mean", timer=ft)
    gx1, gW1 = gpu.flce_backward(xd, Wd, td, lse1, torch.ones(1, device="cuda"), "mean", timer=bt)
    l2, lse2 = gpu.flce_forward(xd, Wd, td, "mean")
    gx2, gW2 = gpu.flce_backward(xd, Wd, td, lse2, torch.ones(1, device="cuda"), "mean")
    torch.cuda.synchronize()
    assert torch.equal(l1, l2) and torch.equal(gx1, gx2) and torch.equal(gW1, gW2)
    fk = [k for k, _ in ft.durations()]
    assert fk == ["fwd_partial", "fwd_combine"]
    bk = contractions(bt)
    # grad_x: 2 output tiles over 2000 vocabulary entries (too few for its own K
    # split), so its work runs as K pieces after an idle main launch
    assert bk == ["bwd_dlogits", "bwd_grad_w", "bwd_grad_x", "tail_pieces", "tail_fixup"], bk
    assert all(ms >= 0 for _, ms in ft.durations() + bt.durations())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_out_of_range_targets(gpu, dtype):
    """Targets outside [0, V) (a caller error the pages leave open; the library's
    contract: the token's loss term and target logit are NaN, its dlogit row gets
    no one-hot term, and nothing is read out of bounds).  Bad targets sit in
    interior tiles (dlogits' unmasked path) and in the ragged last token tile.
    Expected values: lse and every other token's outputs are bit-identical to a run
    with valid targets t0; without the one-hot term a token's dlogit row is
    s softmax(z_i), so grad_x_i = oracle grad_x_i(t0) + s W[t0_i] and
    grad_W = oracle grad_W(t0) + sum over bad tokens of s x_i at row t0_i."""
    N, H, V = 600, 256, 3000
    note(f"[parity] out-of-range targets {dtype}")
    x, W, t0 = make_inputs(N, H, V, dtype, seed=41)
    bad = {5: -1, 100: V, 301: V + 7, 590: -(1 << 40), 599: 1 << 40}
    t = t0.copy()
    for i, v in bad.items():
        t[i] = v
    good = run_hip(gpu, x, W, t0, dtype, "mean")
    got = run_hip(gpu, x, W, t, dtype, "mean")
    idx = np.array(sorted(bad))
    ok = np.setdiff1d(np.arange(N), idx)
    assert math.isnan(got["loss"])
    assert np.all(np.isnan(got["zt"][idx]))
    assert np.array_equal(got["zt"][ok], good["zt"][ok])
    assert np.array_equal(got["lse"], good["lse"])
    assert np.all(np.isfinite(got["gx"])) and np.all(np.isfinite(got["gW"]))
    assert np.array_equal(got["gx"][ok], good["gx"][ok])
    xf, Wf = widen(x, dtype), widen(W, dtype)
    s = 1.0 / N
    ref_gx = oracle.grad_x_rows(xf, Wf, t0, idx, "mean") + s * Wf[t0[idx]]
    _, ref_gW = oracle.backward(xf, Wf, t0, "mean")
    for i in idx:
        ref_gW[t0[i]] += s * xf[i]
    from tests.gpu_util import assert_grad_close
    assert_grad_close(got["gx"][idx], ref_gx, dtype, "grad_x (bad-target rows)")
    assert_grad_close(got["gW"], ref_gW, dtype, "grad_W")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [8000, 16300])
def test_grad_w_balanced(gpu, dtype, V):
    """A grad_W launch of 9 hidden x 32 (V 8000) or 64 (V 16300) vocabulary tiles =
    288 or 576 tiles on 256 workgroups, K = 600 tokens (a ragged last slice): 288
    % 256 = 576 % 256 - 32 = 32 is a multiple of 256 / 8, so the launch is
    balanced -- no round of whole tiles (288) or one (576), then the remaining 288
    or 320 tiles cut evenly along K over the 256 workgroups, each XCD's
    workgroups at one K offset, tiles shared by two workgroups summed through a
    partial-sum slot -- and needs no split-tail launches after it."""
    N, H = 600, 2304
    got = check_case(gpu, N, H, V, dtype, "sum", seed=71, grad_loss=0.8)
    x, W, t = make_inputs(N, H, V, dtype, seed=71)
    xd, Wd, td = to_dev(x, dtype), to_dev(W, dtype), torch.from_numpy(t).cuda()
    bt = gpu.KernelTimer(32)
    gx, gW = gpu.flce_backward(xd, Wd, td, got["raw"]["lse"], torch.tensor([0.8], device="cuda"), "sum", timer=bt)
    torch.cuda.synchronize()
    seq = contractions(bt)
    # (the dlogit launch of 3 x 32 tiles, K = 2304, runs as K pieces)
    i = seq.index("bwd_grad_w")
    assert seq[i + 1] == "bwd_grad_x", seq
    # the same bits again (the shared tiles' sums do not depend on timing)
    gx2, gW2 = gpu.flce_backward(xd, Wd, td, got["raw"]["lse"], torch.tensor([0.8], device="cuda"), "sum")
    torch.cuda.synchronize()
    assert torch.equal(gW.view(torch.int16 if dtype == "bf16" else torch.int32),
                       gW2.view(torch.int16 if dtype == "bf16" else torch.int32))
    assert torch.equal(gx.view(torch.int16 if dtype == "bf16" else torch.int32),
                       gx2.view(torch.int16 if dtype == "bf16" else torch.int32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_whole_slice_splits(gpu, dtype):
    """Split-K work whose K ranges are whole slices ending exactly at the K extent
    (these take the lean copies): one 36864-entry panel of 144 vocabulary tiles,
    512 hidden; the dlogit launch's 4 x 144 (bf16: 1024 tokens) or 2 x 144 (fp32:
    512 tokens) logit tiles leave 64 / 32 tail tiles cut along H into 4 / 8
    pieces, grad_W's 288 tiles are balanced (cut evenly along the tokens over the
    256 workgroups), and grad_x (8 or 4 output tiles) is split 4 ways over the
    vocabulary."""
    N, H, V = (1024 if dtype == "bf16" else 512), 512, 36864
    got = check_case(gpu, N, H, V, dtype, "mean", seed=74, grad_loss=1.1)
    x, W, t = make_inputs(N, H, V, dtype, seed=74)
    xd, Wd, td = to_dev(x, dtype), to_dev(W, dtype), torch.from_numpy(t).cuda()
    bt = gpu.KernelTimer(32)
    gpu.flce_backward(xd, Wd, td, got["raw"]["lse"], torch.tensor([1.1], device="cuda"), "mean", timer=bt)
    torch.cuda.synchronize()
    seq = contractions(bt)
    assert seq == ["bwd_dlogits", "tail_pieces", "tail_fixup", "bwd_grad_w", "bwd_grad_x", "bwd_gx_reduce"], seq


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("panels", [1, 3])
def test_grad_x_balanced(gpu, dtype, panels):
    """A grad_x launch of 16 token x 18 hidden tiles = 288 tiles on 256
    workgroups (no K split of all tiles) is balanced: its tiles cut evenly along K
    (vocabulary) over the workgroups, 32 of them shared by two.  With three
    vocabulary panels (V = 20000 fp32 / 40000 bf16: 8192 / 16384 entries per 128
    MiB panel of 4096 tokens) grad_x runs once per pair of panels: the second
    launch's shared tiles start from the first's float32 sums and are written in
    the output type; the full panels' grad_W launches (18 x 32 or 18 x 64 tiles)
    are balanced after three or one rounds of whole tiles."""
    N, H = 4000, 4608
    V = 3000 if panels == 1 else (20000 if dtype == "f32" else 40000)
    got = check_case(gpu, N, H, V, dtype, "mean", seed=72, grad_loss=1.3)
    x, W, t = make_inputs(N, H, V, dtype, seed=72)
    xd, Wd, td = to_dev(x, dtype), to_dev(W, dtype), torch.from_numpy(t).cuda()
    bt = gpu.KernelTimer(256)
    gpu.flce_backward(xd, Wd, td, got["raw"]["lse"], torch.tensor([1.3], device="cuda"), "mean", timer=bt)
    torch.cuda.synchronize()
    seq = contractions(bt)
    assert seq.count("bwd_grad_x") == (1 if panels == 1 else 2), seq
    assert "bwd_gx_reduce" not in seq, seq
    assert all(b != "tail_pieces" for a, b in zip(seq, seq[1:]) if a == "bwd_grad_x"), seq
    if panels > 1:
        assert seq[:2] == ["bwd_dlogits", "bwd_grad_w"] and seq[2] != "tail_pieces", seq


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("panels", [1, 3])
def test_grad_x_tail_split(gpu, dtype, panels):
    """A grad_x launch of 16 token x 17 hidden tiles = 272 tiles on 256
    workgroups: 272 % 256 = 16 is not a multiple of 256 / 8, so the launch is not
    balanced; the 16 tiles of its partial last round are cut along K (vocabulary)
    into pieces.  With three vocabulary panels (V = 20000 fp32 / 40000 bf16) grad_x
    runs once per pair of panels: the second launch's pieces are added to the
    first's float32 sums and written in the output type."""
    N, H = 4000, 4352
    V = 3000 if panels == 1 else (20000 if dtype == "f32" else 40000)
    got = check_case(gpu, N, H, V, dtype, "mean", seed=72, grad_loss=1.3)
    x, W, t = make_inputs(N, H, V, dtype, seed=72)
    xd, Wd, td = to_dev(x, dtype), to_dev(W, dtype), torch.from_numpy(t).cuda()
    bt = gpu.KernelTimer(256)
    gpu.flce_backward(xd, Wd, td, got["raw"]["lse"], torch.tensor([1.3], device="cuda"), "mean", timer=bt)
    torch.cuda.synchronize()
    seq = contractions(bt)
    after_gx = [seq[i + 1:i + 3] for i, k in enumerate(seq) if k == "bwd_grad_x"]
    assert len(after_gx) == (1 if panels == 1 else 2), seq
    assert all(a == ["tail_pieces", "tail_fixup"] for a in after_gx), seq


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_few_tile_launches(gpu, dtype, reduction):
    """Launches of at most 128 tiles with at least 1024 entries of K run as K pieces
    only, so the idle CUs share their work: the dlogit launch (4 token x 12
    vocabulary tiles, K = H = 1536; targets in the first, a middle and the last,
    ragged vocabulary tile), grad_W (12 x 6 tiles, K = 1024 tokens) and grad_x
    (4 x 6 tiles, K = 3000 vocabulary entries, one panel: no K split of its own)
    each run an idle main launch, their pieces and the fixup."""
    N, H, V = 1024, 1536, 3000
    x, W, t = make_inputs(N, H, V, dtype, seed=75)
    t[:5] = [0, 1500, V - 1, 2816, 255]
    got = check_case(gpu, N, H, V, dtype, reduction, seed=75, grad_loss=1.7, t=t)
    xd, Wd, td = to_dev(x, dtype), to_dev(W, dtype), torch.from_numpy(t).cuda()
    bt = gpu.KernelTimer(32)
    gpu.flce_backward(xd, Wd, td, got["raw"]["lse"], torch.tensor([1.7], device="cuda"), reduction, timer=bt)
    torch.cuda.synchronize()
    seq = contractions(bt)
    assert seq == ["bwd_dlogits", "tail_pieces", "tail_fixup", "bwd_grad_w", "tail_pieces", "tail_fixup",
                   "bwd_grad_x", "tail_pieces", "tail_fixup"], seq


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_dlogits_tail_split(gpu, dtype, reduction):
    """A dlogit launch of 2 token x 137 vocabulary tiles = 274 tiles on 256
    workgroups: the 18 tail tiles (vocabulary 32768 ..) are computed as K
    (hidden) pieces, and the fixup sums them and forms the dlogits, one-hot terms
    included (several targets sit in the tail tiles, one at V - 1); grad_W's 274
    tiles split their tail too."""
    N, H, V = 300, 512, 35000
    x, W, t = make_inputs(N, H, V, dtype, seed=73)
    t[:6] = [32768, 33000, 34000, V - 1, 32900, 34999 - 256]
    got = check_case(gpu, N, H, V, dtype, reduction, seed=73, grad_loss=0.9, t=t)
    xd, Wd, td = to_dev(x, dtype), to_dev(W, dtype), torch.from_numpy(t).cuda()
    bt = gpu.KernelTimer(32)
    gpu.flce_backward(xd, Wd, td, got["raw"]["lse"], torch.tensor([0.9], device="cuda"), reduction, timer=bt)
    torch.cuda.synchronize()
    seq = contractions(bt)
    assert seq[:6] == ["bwd_dlogits", "tail_pieces", "tail_fixup", "bwd_grad_w", "tail_pieces", "tail_fixup"], seq


def _random_cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for k in range(n):
        dtype = ("f32", "bf16")[k % 2]
        reduction = ("mean", "sum")[(k // 2) % 2]
        N = int(rng.integers(1, 700))
        H = int(8 * rng.integers(1, 129))  # a multiple of 16 bytes in either dtype
        V = int(rng.integers(1, 5000))
        gl = float(np.round(rng.uniform(0.5, 2.0), 3))
        cases.append(pytest.param(N, H, V, dtype, reduction, gl, 100 + k, id=f"{dtype}-{reduction}-{N}x{H}x{V}"))
    return cases


@pytest.mark.parametrize("N,H,V,dtype,reduction,grad_loss,seed", _random_cases())
def test_random_shapes(gpu, N, H, V, dtype, reduction, grad_loss, seed):
    """A seeded sweep of small shapes (N in [1, 700), H a multiple of 8 up to 1024, V in
    [1, 5000)), both dtypes and reductions: ragged tiles on every side, any number of
    vocabulary splits and panels, split tails where they occur."""
    check_case(gpu, N, H, V, dtype, reduction, seed=seed, grad_loss=grad_loss)


def _random_panel_cases(n=8, seed=2025):
    rng = np.random.default_rng(seed)
    cases = []
    for k in range(n):
        dtype = ("bf16", "f32")[k % 2]
        reduction = ("mean", "sum")[(k // 2) % 2]
        minimal = k >= n // 2
        N = int(rng.integers(1000, 2049))
        H = int(8 * rng.integers(16, 65))
        # wider than one default 128 MiB panel at 1000 or more tokens (at most 65536
        # bfloat16 or 32768 float32 entries per token)
        V = int(rng.integers(66000, 90000)) if dtype == "bf16" else int(rng.integers(33000, 45000))
        gl = float(np.round(rng.uniform(0.5, 2.0), 3))
        cases.append(pytest.param(N, H, V, dtype, reduction, gl, minimal, 200 + k,
                                  id=f"{dtype}-{reduction}-{N}x{H}x{V}-{'minws' if minimal else 'ws'}"))
    return cases


@pytest.mark.parametrize("N,H,V,dtype,reduction,grad_loss,minimal,seed", _random_panel_cases())
def test_random_shapes_panels(gpu, N, H, V, dtype, reduction, grad_loss, minimal, seed):
    """Seeded shapes large enough for several dlogit panels with the default workspace
    (grad_x over panel pairs where all tokens form one chunk) or, with the minimum
    workspace, many small panels and token chunks with float32 accumulators between
    the launches; the number of dlogit launches is checked."""
    ws = gpu.backward_min_workspace_bytes(N, H, V, torch.bfloat16 if dtype == "bf16" else torch.float32) \
        if minimal else None
    got = check_case(gpu, N, H, V, dtype, reduction, seed=seed, grad_loss=grad_loss, bwd_ws_bytes=ws)
    # the plan really has several panels (and, with the minimum workspace, many)
    x, W, t = make_inputs(N, H, V, dtype, seed=seed)
    xd, Wd, td = to_dev(x, dtype), to_dev(W, dtype), torch.from_numpy(t).cuda()
    bt = gpu.KernelTimer(1024)
    w = None if ws is None else torch.empty(ws, dtype=torch.uint8, device="cuda")
    gpu.flce_backward(xd, Wd, td, got["raw"]["lse"], torch.tensor([grad_loss], device="cuda"), reduction,
                      workspace=w, timer=bt)
    torch.cuda.synchronize()
    n_panels = contractions(bt).count("bwd_dlogits")
    assert n_panels >= (4 if minimal else 2), contractions(bt)
