"""Build the gfx950 shared library ``librgt.so`` in-tree with hipcc.

Run ``python -m router_gemv_top_amd.build`` (or ``__graft_entry__.build()``).
Cross-compiles without a GPU. The library links the HIP runtime by its
soname, so inside a process that already loaded torch's HIP runtime the same
copy is reused.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "librgt.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


TRACE_LIB = os.path.join(PKG, "librgt_trace.so")


def build_cmd(out: str = LIB, extra=()) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # Code object v5: loadable by the HIP runtime that torch bundles.
        "-mcode-object-version=5",
        # Packed fp32 instructions stay off in all device code.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I", INCLUDE, "-I", CSRC,
        os.path.join(CSRC, "rgt.hip"),
        "-Wl,-rpath,/opt/rocm/lib",
        "-o", out, *extra,
    ]


def build(verbose: bool = False, trace: bool = False) -> str:
    """Build librgt.so, or with trace=True the phase-stamping variant
    librgt_trace.so (same ABI; the fused kernel writes per-workgroup clock
    stamps after the regular workspace regions)."""
    lib = TRACE_LIB if trace else LIB
    tmp = lib + ".tmp"
    cmd = build_cmd(tmp, ("-DRGT_TRACE",) if trace else ())
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building librgt.so")
    if verbose and r.stderr.strip():
        sys.stderr.write(r.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True, trace="--trace" in sys.argv))
