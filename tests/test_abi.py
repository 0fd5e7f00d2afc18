"""C-ABI library: loads without a GPU, exports every declared symbol, and rejects
bad arguments before any HIP call (so nothing here touches a device)."""
import ctypes

import pytest

from lm_head_linear_tiled_amd import binding

F32, BF16, MEAN, SUM = 0, 1, 0, 1
OK, NULL, SHAPE, DTYPE, RED, ALIAS, ALIGN, WS, HIPERR, SCRATCH = range(10)


@pytest.fixture(scope="module")
def lib():
    return binding.load()


def test_exports_every_declared_symbol(lib):
    names = binding.header_functions()
    assert set(names) >= {"flce_forward", "flce_backward", "flce_forward_workspace_bytes",
                          "flce_backward_workspace_bytes", "flce_backward_min_workspace_bytes",
                          "flce_status_string", "flce_forward_backward", "flce_forward_backward_workspace_bytes",
                          "flce_forward_timed", "flce_backward_timed"}
    for n in names:
        assert hasattr(lib, n), n


def test_default_build_has_no_tile_clock(lib):
    """The tile clock exists only in measurement builds (FLCE_TILE_CLOCK=1)."""
    assert not hasattr(lib, "flce_tile_clock_read") and not hasattr(lib, "flce_tile_clock_clear")


def test_bench_tile_clock_needs_a_clock_build():
    """bench.py --tile-clock refuses to run without --lib, and with a library that
    has no tile clock (the default build), before touching a device."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for extra, msg in (([], "needs --lib"), (["--lib", binding.LIB_PATH], "was not built with FLCE_TILE_CLOCK")):
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--tile-clock", *extra],
                           capture_output=True, text=True, timeout=300)
        assert r.returncode != 0 and msg in r.stderr, (r.returncode, r.stderr[-500:])


def test_status_strings(lib):
    for code in range(10):
        s = binding.status_string(code)
        assert s.startswith("FLCE_")
    assert "unknown" in binding.status_string(99)


def test_workspace_sizes(lib):
    for (N, H, V) in [(64, 128, 1000), (1269, 1000, 10000), (4096, 4096, 128256), (32768, 4096, 128256)]:
        for dt in (F32, BF16):
            f = lib.flce_forward_workspace_bytes(N, H, V, dt)
            b = lib.flce_backward_workspace_bytes(N, H, V, dt)
            bmin = lib.flce_backward_min_workspace_bytes(N, H, V, dt)
            assert f > 0 and b > 0 and 0 < bmin <= b
    assert lib.flce_forward_workspace_bytes(0, 4, 4, F32) == 0
    assert lib.flce_backward_workspace_bytes(4, 4, 4, 5) == 0
    assert lib.flce_backward_min_workspace_bytes(4, -1, 4, F32) == 0


# Fake, well-separated, 16-byte aligned addresses: every call below fails its
# checks before a pointer is used.
X, Wp, T, LOSS, LSE, ZT, WSP, GX, GW, GL = (0x10_0000_0000 + i * 0x1_0000_0000 for i in range(10))


def fwd(lib, x=X, W=Wp, t=T, N=64, H=128, V=1000, dt=F32, red=MEAN, loss=LOSS, lse=LSE, zt=ZT, ws=WSP,
        nws=None):
    if nws is None:
        nws = lib.flce_forward_workspace_bytes(N, H, V, dt) if N > 0 and H > 0 and V > 0 else 0
    return lib.flce_forward(x, W, t, N, H, V, dt, red, loss, lse, zt, ws, nws, None)


def bwd(lib, x=X, W=Wp, t=T, lse=LSE, gl=GL, N=64, H=128, V=1000, dt=F32, red=MEAN, gx=GX, gw=GW, ws=WSP,
        nws=None):
    if nws is None:
        nws = lib.flce_backward_workspace_bytes(N, H, V, dt) if N > 0 and H > 0 and V > 0 else 0
    return lib.flce_backward(x, W, t, lse, gl, N, H, V, dt, red, gx, gw, ws, nws, None)


def test_forward_rejects(lib):
    assert fwd(lib, x=None) == NULL
    assert fwd(lib, t=None) == NULL
    assert fwd(lib, loss=None) == NULL
    assert fwd(lib, lse=None) == NULL
    assert fwd(lib, N=0) == SHAPE
    assert fwd(lib, V=-3) == SHAPE
    assert fwd(lib, H=1 << 31) == SHAPE
    assert fwd(lib, dt=2) == DTYPE
    assert fwd(lib, red=2) == RED
    assert fwd(lib, x=X + 8) == ALIGN
    assert fwd(lib, W=Wp + 4) == ALIGN
    assert fwd(lib, H=130) == ALIGN            # 130 * 4 bytes is not a multiple of 16
    assert fwd(lib, H=132, dt=BF16) == ALIGN   # 132 * 2 bytes is not a multiple of 16
    assert fwd(lib, lse=X + 64) == ALIAS       # lse inside x
    assert fwd(lib, zt=LSE + 16) == ALIAS      # target_logit overlaps lse
    assert fwd(lib, loss=WSP + 4) == ALIAS     # loss inside the workspace
    assert fwd(lib, ws=T) == ALIAS             # workspace over the targets
    assert fwd(lib, ws=None) == WS
    assert fwd(lib, nws=16) == WS


def test_backward_rejects(lib):
    assert bwd(lib, lse=None) == NULL
    assert bwd(lib, gl=None) == NULL
    assert bwd(lib, gx=None) == NULL
    assert bwd(lib, gw=None) == NULL
    assert bwd(lib, N=-1) == SHAPE
    assert bwd(lib, dt=9) == DTYPE
    assert bwd(lib, red=-1) == RED
    assert bwd(lib, x=X + 2) == ALIGN
    assert bwd(lib, gx=Wp) == ALIAS            # grad_x over W
    assert bwd(lib, gw=GX + 128) == ALIAS      # grad_W overlaps grad_x
    assert bwd(lib, gx=LSE) == ALIAS           # grad_x over lse
    assert bwd(lib, ws=GW + 64) == ALIAS       # workspace over grad_W
    assert bwd(lib, ws=None) == WS
    assert bwd(lib, nws=lib.flce_backward_min_workspace_bytes(64, 128, 1000, F32) - 1) == WS


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 8)
    with pytest.raises(ValueError):
        binding.flce_forward(x, torch.zeros(5, 8), torch.zeros(4, dtype=torch.int64))
    with pytest.raises(TypeError):
        binding.flce_forward(x.double(), torch.zeros(5, 8).double(), torch.zeros(4, dtype=torch.int64))


def fb(lib, x=X, W=Wp, t=T, N=64, H=128, V=1000, dt=F32, red=MEAN, gl=GL, loss=LOSS, lse=LSE, gx=GX, gw=GW,
       ws=WSP, nws=None):
    if nws is None:
        nws = lib.flce_forward_backward_workspace_bytes(N, H, V, dt) if N > 0 and H > 0 and V > 0 else 0
    return lib.flce_forward_backward(x, W, t, N, H, V, dt, red, gl, loss, lse, gx, gw, ws, nws, None)


def test_forward_backward_rejects(lib):
    assert fb(lib, x=None) == NULL
    assert fb(lib, lse=None) == NULL
    assert fb(lib, gw=None) == NULL
    assert fb(lib, N=0) == SHAPE
    assert fb(lib, dt=4) == DTYPE
    assert fb(lib, red=3) == RED
    assert fb(lib, W=Wp + 8) == ALIGN
    assert fb(lib, lse=GX + 32) == ALIAS       # lse inside grad_x
    assert fb(lib, gl=LOSS) == ALIAS           # grad_loss is the loss output
    assert fb(lib, ws=X) == ALIAS
    assert fb(lib, ws=None) == WS
    assert fb(lib, nws=255) == WS
    n = lib.flce_forward_backward_workspace_bytes(64, 128, 1000, F32)
    assert n >= 256 + lib.flce_forward_workspace_bytes(64, 128, 1000, F32)
    assert n >= 256 + lib.flce_backward_workspace_bytes(64, 128, 1000, F32)


def bch(lib, x=X, W=Wp, t=T, lse=LSE, gl=GL, N=64, H=128, V=1000, dt=F32, red=MEAN, chunk=256, gx=GX, gw=GW,
        ws=WSP, nws=None):
    if nws is None:
        nws = lib.flce_backward_chunked_workspace_bytes(N, H, V, dt, chunk) if min(N, H, V, chunk) > 0 else 0
    return lib.flce_backward_chunked(x, W, t, lse, gl, N, H, V, dt, red, chunk, gx, gw, ws, nws, None, None)


def test_backward_chunked_workspace_sizes(lib):
    # one chunk of every token over the whole vocabulary; many chunks need the
    # float32 grad_W accumulator for bfloat16 only
    N, H, V = 4096, 4096, 128256
    one = lib.flce_backward_chunked_workspace_bytes(N, H, V, BF16, N)
    assert one >= 2 * N * ((V + 255) // 256 * 256)
    many = lib.flce_backward_chunked_workspace_bytes(N, H, V, BF16, 256)
    assert many >= 2 * 256 * V + 4 * V * H
    assert lib.flce_backward_chunked_workspace_bytes(N, H, V, F32, 256) < 4 * V * H
    assert lib.flce_backward_chunked_workspace_bytes(N, H, V, BF16, 10 ** 9) == one  # capped at N
    assert lib.flce_backward_chunked_workspace_bytes(N, H, V, BF16, 1) == many       # rounded up to 256
    assert lib.flce_backward_chunked_workspace_bytes(N, H, V, BF16, 0) == 0
    assert lib.flce_backward_chunked_workspace_bytes(0, H, V, BF16, 256) == 0


def test_backward_chunked_rejects(lib):
    assert bch(lib, chunk=0) == SHAPE
    assert bch(lib, chunk=-5) == SHAPE
    assert bch(lib, lse=None) == NULL
    assert bch(lib, gw=None) == NULL
    assert bch(lib, N=0) == SHAPE
    assert bch(lib, dt=3) == DTYPE
    assert bch(lib, red=7) == RED
    assert bch(lib, W=Wp + 4) == ALIGN
    assert bch(lib, gx=T) == ALIAS
    assert bch(lib, ws=GX + 16) == ALIAS
    assert bch(lib, ws=None) == WS
    assert bch(lib, nws=lib.flce_backward_chunked_workspace_bytes(64, 128, 1000, F32, 256) - 1) == WS


def test_backward_plan_shapes(lib):
    """The panel shape the backward picks, read off the workspace it asks for
    (panel + float32 accumulators), at the headline and at N=32768, V=32000."""
    MB = 1 << 20
    # headline: panels of 4096 tokens x 16384 vocabulary (128 MB bf16), two of them
    # kept at once (all tokens form one chunk: grad_x runs once per pair of panels)
    # + grad_x accumulator [N, H] f32 + the float32 pieces of the split tail of the
    # last panel's grad_W launch (53 x 16 = 848 tiles on 256 workgroups: 80 tail
    # tiles in 3 pieces each)
    assert lib.flce_backward_workspace_bytes(4096, 4096, 128256, BF16) == \
        2 * 128 * MB + 4096 * 4096 * 4 + 80 * 3 * 256 * 256 * 4
    # 8192 x 8192 panel (not 32768 x 2048, whose grad_W launches would fill half the CUs)
    # + grad_x accumulator [N, H] + grad_W accumulator [8192, H]
    assert lib.flce_backward_workspace_bytes(32768, 4096, 32000, BF16) == \
        128 * MB + 32768 * 4096 * 4 + 8192 * 4096 * 4
    # a single panel covers a smaller problem: no accumulators; its grad_x launches
    # would fill half the CUs, so their vocabulary is split in two (float32 partials)
    assert lib.flce_backward_workspace_bytes(2048, 4096, 32000, BF16) == 2048 * 32000 * 2 + 2 * 2048 * 4096 * 4


def test_row_length_limits(lib):
    """A 256-row operand tile is addressed through one 2 GiB buffer range, so rows of
    more than 8 MiB (H of x and W, padded V of a dlogit panel) are refused."""
    MiB = 1 << 20
    assert lib.flce_forward_workspace_bytes(64, 4 * MiB, 1000, BF16) > 0      # 8 MiB rows: allowed
    assert lib.flce_forward_workspace_bytes(64, 4 * MiB + 8, 1000, BF16) == 0
    assert lib.flce_backward_workspace_bytes(64, 2 * MiB + 4, 1000, F32) == 0
    assert lib.flce_backward_workspace_bytes(64, 128, 4 * MiB, BF16) > 0
    assert lib.flce_backward_workspace_bytes(64, 128, 4 * MiB + 1, BF16) == 0  # padded to 256 entries
    assert lib.flce_backward_chunked_workspace_bytes(64, 128, 2 * MiB + 1, F32, 256) == 0
    assert fwd(lib, H=4 * MiB + 8, dt=BF16) == SHAPE
    # 2^22 token tiles x 2^9 vocabulary tiles = 2^31 logit tiles: not countable in 32 bits
    assert lib.flce_forward_workspace_bytes(1 << 30, 128, 1 << 17, BF16) == 0
    assert lib.flce_forward_workspace_bytes(1 << 30, 128, (1 << 17) - 256, BF16) > 0
    assert bwd(lib, V=2 * MiB + 1, nws=1 << 40) == SHAPE


def test_noalloc_forward_limits_and_rejects(lib):
    """flce_forward_noalloc checks its arguments like flce_forward and refuses sizes
    whose forward workspace exceeds the static scratch, before any HIP call."""
    MiB = 1 << 20
    for V in (1000, 128256, 262208):
        nmax = lib.flce_forward_noalloc_max_tokens(V)
        assert nmax > 400000
        assert lib.flce_forward_workspace_bytes(nmax, 128, V, BF16) <= 16 * MiB
        assert lib.flce_forward_workspace_bytes(nmax + 1, 128, V, BF16) > 16 * MiB
    assert lib.flce_forward_noalloc_max_tokens(0) == 0

    def na(x=X, W=Wp, t=T, N=64, H=128, V=1000, dt=F32, red=MEAN, loss=LOSS, lse=LSE, zt=ZT):
        return lib.flce_forward_noalloc(x, W, t, N, H, V, dt, red, loss, lse, zt, None)
    assert na(x=None) == NULL
    assert na(lse=None) == NULL
    assert na(N=0) == SHAPE
    assert na(dt=2) == DTYPE
    assert na(red=5) == RED
    assert na(W=Wp + 4) == ALIGN
    assert na(lse=X + 64) == ALIAS
    assert na(N=lib.flce_forward_noalloc_max_tokens(1000) + 1) == SCRATCH
    assert "static scratch" in binding.status_string(SCRATCH)


def test_backward_atomic_workspace_and_rejects(lib):
    """flce_backward_atomic: 256 dlogit tiles of 256 x 256, plus float32 [N, H] and
    [V, H] accumulators for bfloat16 (float32 accumulates in place); argument checks
    before any HIP call."""
    N, H, V = 4096, 4096, 128256
    assert lib.flce_backward_atomic_workspace_bytes(N, H, V, BF16) == 256 * 256 * 256 * 2 + 4 * N * H + 4 * V * H
    assert lib.flce_backward_atomic_workspace_bytes(N, H, V, F32) == 256 * 256 * 256 * 4
    assert lib.flce_backward_atomic_workspace_bytes(0, H, V, F32) == 0

    def ba(x=X, W=Wp, t=T, lse=LSE, gl=GL, N=64, H=128, V=1000, dt=F32, red=MEAN, gx=GX, gw=GW, ws=WSP, nws=None):
        if nws is None:
            nws = lib.flce_backward_atomic_workspace_bytes(N, H, V, dt) if min(N, H, V) > 0 else 0
        return lib.flce_backward_atomic(x, W, t, lse, gl, N, H, V, dt, red, gx, gw, ws, nws, None, None)
    assert ba(lse=None) == NULL
    assert ba(gw=None) == NULL
    assert ba(N=0) == SHAPE
    assert ba(dt=3) == DTYPE
    assert ba(red=9) == RED
    assert ba(x=X + 4) == ALIGN
    assert ba(gx=Wp) == ALIAS
    assert ba(ws=GX + 16) == ALIAS
    assert ba(ws=None) == WS
    assert ba(nws=lib.flce_backward_atomic_workspace_bytes(64, 128, 1000, F32) - 1) == WS
