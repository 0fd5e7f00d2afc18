#!/usr/bin/env python3
"""Benchmark of fused linear + cross-entropy on one MI355X.

One step = flce_forward + flce_backward (loss, lse, grad_x, grad_W) over the
Llama-3 head workload (V=128256, H=4096, N=4096 tokens, bf16 inputs, mean),
inputs resident in HBM.  Prints one JSON line with the throughput (8NHV flop
per step), forward time, per-kernel timings from HIP events recorded between
the library's launches, the roofline of the dominant kernel and the CPU oracle
timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd+bwd ms & TFLOP/s (8NHV) at V=128256 H=4096 N=4096 bf16; fwd ms"


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_4k")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target length of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", choices=["panels", "chunked", "atomic"], default="panels",
                    help="panels: flce_backward (bounded dlogit panels, the default); chunked: "
                         "flce_backward_chunked, token chunks over the whole vocabulary; atomic: "
                         "flce_backward_atomic, float32 atomic accumulation of both gradients (the last two "
                         "for comparison)")
    ap.add_argument("--chunk-tokens", type=int, default=1024, help="tokens per chunk for --backward chunked")
    ap.add_argument("--lib", default=None,
                    help="load this build of libflce.so instead of the package's (a variant built with "
                         "python -m lm_head_linear_tiled_amd.build --define NAME=VALUE --out PATH)")
    ap.add_argument("--workspace-mb", type=float, default=None,
                    help="backward workspace in MiB instead of the library's default size (the planner then "
                         "uses the largest dlogit panels whose plan fits)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (3 times), to scale the HBM counters")
    ap.add_argument("--dma-calibration", action="store_true",
                    help="only run the forward on one 256 x 256 tile with H = 65536 (3 times): one workgroup "
                         "reads x and W (32 MiB each) once through the global -> LDS copies, to check that the "
                         "counters scaled by the copy calibration count those copies' bytes")
    ap.add_argument("--tile-clock", action="store_true",
                    help="only report where the forward's and the backward kernels' cycles go, per output "
                         "tile (first K slice, steady K slices, epilogue, gap to the next tile) at N = 4096 and "
                         "2048, H = 4096, V = 32768, bf16 (launches without split tails); needs --lib with a build "
                         "made with --define FLCE_TILE_CLOCK=1")
    return ap.parse_args()


KERNEL_SOURCES = ["lm_head_linear_tiled_amd/csrc/gemm_core.h", "lm_head_linear_tiled_amd/csrc/flce_kernels.hip",
                  "lm_head_linear_tiled_amd/csrc/flce_launch.h", "lm_head_linear_tiled_amd/csrc/flce_api.cpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "flce_llama3_4k_bf16_traffic.json")


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed counter profile, or None
    when there is none for this workload or the kernels changed since it was taken."""
    try:
        import json as _j
        prof = _j.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if prof.get("source_hash") != kernel_source_hash() or prof.get("workload") != workload:
        return None
    k = prof.get("kernels", {}).get(kernel)
    return None if k is None else int(k["hbm_bytes_per_launch"])


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}), flush=True)


def dma_calibration():
    import torch

    from lm_head_linear_tiled_amd import binding
    N, H, V = 256, 65536, 256
    g = torch.Generator(device="cpu").manual_seed(0)
    x = torch.randn(N, H, generator=g).to(torch.bfloat16).cuda()
    W = (torch.randn(V, H, generator=g) / 256).to(torch.bfloat16).cuda()
    t = torch.randint(0, V, (N,), generator=g).cuda()
    for _ in range(3):
        binding.flce_forward(x, W, t, "mean")
    torch.cuda.synchronize()
    print(json.dumps({"kernel": "fwd_partial", "compulsory_bytes_read": 2 * N * H * 2 + 8 * N, "launches": 3}),
          flush=True)


def tile_clock(lib_path):
    """Per-tile cycle split of the forward and of the last dlogit, grad_W and grad_x
    launches of one backward (a build with FLCE_TILE_CLOCK records the shader clock
    at each item's start, after its first K slice, after its last K slice and after
    its epilogue)."""
    import ctypes

    import numpy as np
    import torch

    from lm_head_linear_tiled_amd import binding
    from lm_head_linear_tiled_amd.inputs import make_inputs
    if lib_path is None:
        sys.exit("--tile-clock needs --lib: a build made with --define FLCE_TILE_CLOCK=1")
    binding.LIB_PATH = os.path.abspath(lib_path)
    lib = binding.load()
    if not hasattr(lib, "flce_tile_clock_read"):
        sys.exit(f"{lib_path} was not built with FLCE_TILE_CLOCK=1")
    lib.flce_tile_clock_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.flce_tile_clock_read.restype = ctypes.c_int
    lib.flce_tile_clock_clear.argtypes = []
    lib.flce_tile_clock_clear.restype = ctypes.c_int
    rec = np.zeros((4, 256, 64, 5), np.uint64)
    ideal = 256 * 256 * 64 * 2 / 4096  # cycles of one bf16 K slice at the CU's MFMA peak (4096 flop/clock)

    def report(kind, name, N, H, V):
        r = rec[kind].astype(np.int64)
        items, gaps = [], []
        for b in range(256):
            for j in range(64):
                if r[b, j, 3] == 0:
                    continue
                nkt = int(r[b, j, 4])
                items.append((nkt, r[b, j, 1] - r[b, j, 0], (r[b, j, 2] - r[b, j, 1]) / max(nkt - 1, 1),
                              r[b, j, 3] - r[b, j, 2]))
                if j + 1 < 64 and r[b, j + 1, 3] != 0:
                    gaps.append(r[b, j + 1, 0] - r[b, j, 3])
        a = np.array(items, dtype=np.float64)
        nkt = float(np.median(a[:, 0]))
        first, steady, epi = (float(np.median(a[:, c])) for c in (1, 2, 3))
        gap = float(np.median(gaps)) if gaps else 0.0
        tile = first + (nkt - 1) * steady + epi + gap
        print(json.dumps({"kernel": name, "N": N, "H": H, "V": V, "items": len(items),
                          "items_per_workgroup": round(len(items) / 256, 2), "k_slices": nkt,
                          "first_slice": first, "steady_slice": round(steady, 1), "epilogue": epi,
                          "gap": gap if gaps else None, "ideal_slice": ideal,
                          "steady_mfma_frac": round(ideal / steady, 4),
                          "tile_mfma_frac": round(nkt * ideal / tile, 4),
                          "unit": "shader clock cycles (medians over items)"}), flush=True)

    for N, H, V in ((4096, 4096, 32768), (2048, 4096, 32768)):
        x, W, t = make_inputs(N, H, V, "bf16", seed=0)
        xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        Wd = torch.from_numpy(W.view(np.int16)).view(torch.bfloat16).cuda()
        td = torch.from_numpy(t).cuda()
        gl = torch.ones(1, dtype=torch.float32, device="cuda")
        for _ in range(3):
            _, lse = binding.flce_forward(xd, Wd, td, "mean")
            binding.flce_backward(xd, Wd, td, lse, gl, "mean")
        torch.cuda.synchronize()
        assert lib.flce_tile_clock_clear() == 0
        binding.flce_forward(xd, Wd, td, "mean")
        torch.cuda.synchronize()
        assert lib.flce_tile_clock_read(rec.ctypes.data, rec.nbytes) == 0
        report(3, "fwd_partial", N, H, V)
        assert lib.flce_tile_clock_clear() == 0
        binding.flce_backward(xd, Wd, td, lse, gl, "mean")
        torch.cuda.synchronize()
        assert lib.flce_tile_clock_read(rec.ctypes.data, rec.nbytes) == 0
        for kind, name in ((2, "bwd_dlogits"), (0, "bwd_grad_w"), (1, "bwd_grad_x")):
            report(kind, name, N, H, V)


def cpu_baseline(x, W, t, dtype, H, V, target_s):
    """Time the CPU oracle (forward, then backward) on a token sample of the workload."""
    import numpy as np

    import oracle
    from lm_head_linear_tiled_amd.inputs import widen
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        cores = max(int(i.get("num_threads", 1)) for i in info)
        blas = ", ".join(f"{i.get('internal_api')} {i.get('version')} ({i.get('architecture')})" for i in info)
    except Exception:  # threadpoolctl missing: fall back to the affinity mask
        cores = len(os.sched_getaffinity(0))
    cpu_model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    Wf = widen(W, dtype)

    def run(n):
        xs = widen(x[:n], dtype)
        ts = t[:n]
        t0 = time.perf_counter()
        oracle.forward(xs, Wf, ts, "mean")
        oracle.backward(xs, Wf, ts, "mean")
        return time.perf_counter() - t0

    n, secs = 16, run(16)
    while secs < target_s / 4 and n < len(t):  # grow the sample until it is timeable
        n = min(len(t), 4 * n)
        secs = run(n)
    if secs < target_s and n < len(t):
        n = int(min(len(t), n * target_s / secs))
        secs = run(n)
    tflops = 8.0 * n * H * V / secs / 1e12
    return {"value": round(tflops, 4), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model, "blas": blas,
            "sample": f"{n} of {len(t)} tokens x full V={V}, H={H}: oracle.forward then oracle.backward "
                      f"(float64 numpy, logits materialised per token chunk), {secs:.1f} s",
            "seconds": round(secs, 2), "tokens": n}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.dma_calibration:
        dma_calibration()
        return
    if args.tile_clock:
        tile_clock(args.lib)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported (the path has no multi-GPU sharding)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from lm_head_linear_tiled_amd import binding, roofline
    from lm_head_linear_tiled_amd.inputs import WORKLOADS, make_inputs
    if args.lib:
        binding.LIB_PATH = os.path.abspath(args.lib)

    w = WORKLOADS[args.workload]
    N, H, V, dtype = w.N, w.H, w.V, w.dtype
    red = "mean"
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    x, W, t = make_inputs(N, H, V, dtype, seed=0)
    if dtype == "bf16":
        xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        Wd = torch.from_numpy(W.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        xd, Wd = torch.from_numpy(x).to(dev), torch.from_numpy(W).to(dev)
    td = torch.from_numpy(t).to(dev)
    gl = torch.ones(1, dtype=torch.float32, device=dev)
    fws = torch.empty(binding.forward_workspace_bytes(N, H, V, tdt), dtype=torch.uint8, device=dev)
    if args.backward == "chunked":
        nbws = binding.backward_chunked_workspace_bytes(N, H, V, tdt, args.chunk_tokens)
    elif args.backward == "atomic":
        nbws = binding.backward_atomic_workspace_bytes(N, H, V, tdt)
    else:
        nbws = binding.backward_workspace_bytes(N, H, V, tdt)
    if args.workspace_mb is not None:
        nbws = int(args.workspace_mb * (1 << 20))
    bws = torch.empty(nbws, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()

    def step(ft=None, bt=None):
        loss, lse = binding.flce_forward(xd, Wd, td, red, workspace=fws, timer=ft)
        if args.backward == "chunked":
            gx, gW = binding.flce_backward_chunked(xd, Wd, td, lse, gl, red, chunk_tokens=args.chunk_tokens,
                                                   workspace=bws, timer=bt)
        elif args.backward == "atomic":
            gx, gW = binding.flce_backward_atomic(xd, Wd, td, lse, gl, red, workspace=bws, timer=bt)
        else:
            gx, gW = binding.flce_backward(xd, Wd, td, lse, gl, red, workspace=bws, timer=bt)
        return loss, gx, gW

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    n_bwd_launches = 3 * 256  # covers every panel and chunk launch at these sizes
    ftimers = [binding.KernelTimer(4) for _ in range(args.steps)]
    btimers = [binding.KernelTimer(n_bwd_launches + 1) for _ in range(args.steps)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    res = None
    for k in range(args.steps):
        res = None  # a step's outputs are dropped before the next step allocates its own
        res = step(ftimers[k], btimers[k])
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = e0.elapsed_time(e1) / args.steps

    # forward alone
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    f0.record()
    for _ in range(args.steps):
        binding.flce_forward(xd, Wd, td, red, workspace=fws)
    f1.record()
    torch.cuda.synchronize()
    fwd_ms = f0.elapsed_time(f1) / args.steps
    # peak device memory of one step on its own: inputs, workspaces and that step's outputs
    res = None
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    res = step()
    torch.cuda.synchronize()
    peak_mem = torch.cuda.max_memory_allocated()
    res = None

    # per-kernel durations from the events recorded inside the timed steps; the
    # split-tail launches (K pieces and fixup of a launch's partial last round)
    # finish the contraction launched just before them and count towards it
    per = {}
    with_tail = {}
    for tm in ftimers + btimers:
        parent = None
        for name, ms in tm.durations():
            per.setdefault(name, []).append(ms)
            if name in ("tail_pieces", "tail_fixup"):
                if parent is not None:
                    with_tail[parent] = with_tail.get(parent, 0.0) + ms
            else:
                parent = name
                with_tail[name] = with_tail.get(name, 0.0) + ms
    fl_kind = {"fwd_partial": roofline.fwd_flops(N, H, V)}
    for k in ("bwd_dlogits", "bwd_grad_w", "bwd_grad_x"):
        fl_kind[k] = roofline.fwd_flops(N, H, V)  # each backward contraction sums to 2NHV over a step
    fl_kind["bwd_atomic"] = 3 * roofline.fwd_flops(N, H, V)  # the fused atomic kernel does all three
    kernels = {}
    for name, ms in per.items():
        tot = sum(ms) / args.steps
        kernels[name] = {"launches_per_step": len(ms) // args.steps, "avg_ms": round(sum(ms) / len(ms), 4),
                         "ms_per_step": round(tot, 4)}
        if name in fl_kind:
            # the contraction's whole 2NHV share over its own launches and its split tails
            full = with_tail[name] / args.steps
            kernels[name]["tflops"] = round(fl_kind[name] / (full * 1e-3) / 1e12, 2)
            if full > tot * 1.0000001:
                kernels[name]["ms_per_step_with_tail"] = round(full, 4)
    dom = max((k for k in kernels if k in fl_kind), key=lambda k: with_tail[k])
    launches = kernels[dom]["launches_per_step"]
    flops_per_launch = fl_kind[dom] / launches
    # average duration per launch, the split tail's share spread over the launches
    dom_avg_ms = with_tail[dom] / args.steps / launches
    achieved = flops_per_launch / (dom_avg_ms * 1e-3) / 1e12
    peak = roofline.PEAK_TFLOPS[dtype]

    total_flops = roofline.fwdbwd_flops(N, H, V)
    value = total_flops / (ms_step * 1e-3) / 1e12
    out = {
        "metric": METRIC if args.workload == "llama3_4k" else
        f"fwd+bwd ms & TFLOP/s (8NHV) at V={V} H={H} N={N} {dtype}; fwd ms",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (x~N(0,1), W~N(0,1/sqrt(H)), targets uniform, seed 0)",
        "config": {"workload": f"{args.workload}: LM head V={V} H={H} N={N} {dtype} mean, forward+backward",
                   "N": N, "H": H, "V": V, "reduction": red,
                   "backward": {"panels": "panels", "atomic": "atomic"}.get(args.backward,
                                                                             f"chunked {args.chunk_tokens} tokens"),
                   "backward_workspace_bytes": int(nbws)},
        "fwd_ms": round(fwd_ms, 4),
        "fwd_tflops": round(roofline.fwd_flops(N, H, V) / (fwd_ms * 1e-3) / 1e12, 2),
        "fwdbwd_frac_of_peak": round(value / peak, 4),
        "fwd_frac_of_peak": round(roofline.fwd_flops(N, H, V) / (fwd_ms * 1e-3) / 1e12 / peak, 4),
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
        "peak_mem_bytes": int(peak_mem),
        "kernels": kernels,
        "roofline": {"bound": "mfma", "kernel": dom, "avg_launch_ms": round(dom_avg_ms, 4),
                     "tail_included": "ms_per_step_with_tail" in kernels[dom],
                     "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(dom, args.workload) if not args.lib else None,
                     "traffic_scope": "bytes past the L2 (L2 misses, last-level-cache hits included): rocprofv3 "
                                      "FETCH_SIZE and WRITE_SIZE per launch, scaled by what they read for a plain "
                                      "1 GiB device copy",
                     "flops_per_launch": flops_per_launch, "kernel_source_hash": kernel_source_hash()},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, W, t, dtype, H, V, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
