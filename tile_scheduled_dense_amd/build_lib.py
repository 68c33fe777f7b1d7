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
# the C ABI and planning, the layout introspection, and one translation unit per
# input type for the GEMM kernels (compiled in parallel, then linked)
SOURCES = [os.path.join(CSRC, f) for f in ("tile_gemm.hip", "layout.hip", "launch_bf16.hip", "launch_f16.hip",
                                           "launch_f32.hip")]
BUILD_DIR = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops are kept out of the generated code on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _quiet(text: str) -> str:
    return "\n".join(l for l in text.splitlines()
                     if l.strip() and "packed-fp32-ops" not in l and "not a recognized feature" not in l)


def build(verbose: bool = False, extra=(), log: str | None = None) -> str:
    """Compile every source to an object (in parallel), then link the shared library.
    extra: more compiler flags (e.g. resource-usage remarks); log: a file that receives
    everything the compiler printed."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    t = time.time()
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        cmd = [HIPCC, *FLAGS, *extra, "-c", "-o", obj, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    outputs, failed = [], []
    for src, obj, proc in jobs:
        out, _ = proc.communicate()
        outputs.append(out)
        if proc.returncode != 0:
            failed.append(src)
            sys.stderr.write(out)
    if log:
        with open(log, "w") as f:
            f.write("".join(outputs))
    if failed:
        raise RuntimeError(f"hipcc failed on {', '.join(os.path.basename(f) for f in failed)}")
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp", *[o for _, o, _ in jobs]]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("linking libtile_gemm.so failed")
    noisy = _quiet("".join(outputs) + r.stdout + r.stderr)
    if verbose and noisy:
        print(noisy)
    os.replace(LIB + ".tmp", LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t:.1f}s", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
