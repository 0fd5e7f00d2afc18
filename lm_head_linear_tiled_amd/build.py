"""Build libflce.so (the HIP library behind include/flce.h) in-tree for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libflce.so")
SOURCES = ["csrc/flce_kernels.hip", "csrc/flce_api.cpp"]
HEADERS = ["csrc/gemm_core.h", "csrc/flce_launch.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 ops are kept out of the generated device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False, defines=(), out: str | None = None) -> str:
    """Compile every source into libflce.so (always recompiles).

    defines: extra NAME=VALUE macros (the tuning knobs the sources declare with
    #ifndef, e.g. FLCE_PANEL_MB=64); out: where to put the library instead of the
    package directory (measurement variants)."""
    lib = os.path.abspath(out) if out else LIB
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    tmp = lib + ".tmp"
    cmd = [HIPCC, *FLAGS, *[f"-D{d}" for d in defines], "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(PKG, "csrc"), *[os.path.join(PKG, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description="build libflce.so for gfx950")
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--define", action="append", default=[], metavar="NAME=VALUE",
                    help="extra macro for a measurement variant (repeatable)")
    ap.add_argument("--out", default=None, help="output path (default: the package directory)")
    a = ap.parse_args()
    print(build(verbose=a.verbose, defines=a.define, out=a.out))
