"""Build libtile_gemm.so in-tree with hipcc for gfx950.

Usage: python -m tile_scheduled_dense_amd.build_lib [-v]
"""
from __future__ import annotations

import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libtile_gemm.so")
SOURCES = [os.path.join(CSRC, f) for f in ("tile_gemm.hip", "layout.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU ops are kept out of the generated code on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(verbose: bool = False, extra=()) -> str:
    cmd = [HIPCC, *FLAGS, *extra, "-o", LIB + ".tmp", *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    t = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libtile_gemm.so")
    noisy = [l for l in (r.stdout + r.stderr).splitlines()
             if l.strip() and "packed-fp32-ops" not in l and "not a recognized feature" not in l]
    if verbose and noisy:
        print("\n".join(noisy))
    os.replace(LIB + ".tmp", LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t:.1f}s", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
