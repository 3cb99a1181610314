"""Build the gfx950 shared library ``librgt.so`` in-tree with hipcc.

Run ``python -m router_gemv_top_amd.build`` (or ``__graft_entry__.build()``).
Cross-compiles without a GPU. The host side and the fused kernel's instances
(one translation unit per expert-count bucket) compile in parallel to objects
under ``_build/`` and are linked into one library. The library links the HIP
runtime by its soname, so inside a process that already loaded torch's HIP
runtime the same copy is reused.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "librgt.so")
TRACE_LIB = os.path.join(PKG, "librgt_trace.so")
OBJ_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"
NV_BUCKETS = (2, 4, 8, 14, 16)


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # Code object v5: loadable by the HIP runtime that torch bundles.
        "-mcode-object-version=5",
        # Packed fp32 instructions stay off in all device code.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I", INCLUDE, "-I", CSRC,
    ]


def units(trace: bool):
    """(source, object, extra defines) of every translation unit."""
    tag = "trace" if trace else "rel"
    d = os.path.join(OBJ_DIR, tag)
    extra = ["-DRGT_TRACE"] if trace else []
    # the chain's kernels: their first eight arguments preloaded into scalar
    # registers at dispatch (those that take scalars first; the rest read the
    # argument block as before)
    out = [(os.path.join(CSRC, "rgt.hip"), os.path.join(d, "rgt.o"),
            extra + ["-mllvm", "-amdgpu-kernarg-preload-count=8"])]
    for norm in (0, 1):
        for nv in NV_BUCKETS:
            name = f"fused_norm_nv{nv}.o" if norm else f"fused_nv{nv}.o"
            # the fused kernels' ten leading scalar arguments (the tile's
            # operands) are preloaded into scalar registers at dispatch
            out.append((os.path.join(CSRC, "fused_inst.hip"), os.path.join(d, name),
                        extra + [f"-DRGT_NV={nv}", f"-DRGT_NORM={norm}", "-mllvm",
                                 "-amdgpu-kernarg-preload-count=10"]))
    # the router + shared-expert kernel's eight leading scalar arguments
    out.append((os.path.join(CSRC, "shared_inst.hip"), os.path.join(d, "shared_inst.o"),
                extra + ["-mllvm", "-amdgpu-kernarg-preload-count=8"]))
    return out


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed: " + " ".join(cmd[-6:]))
    if verbose and r.stderr.strip():
        sys.stderr.write(r.stderr)


def build(verbose: bool = False, trace: bool = False, jobs: int = 0) -> str:
    """Build librgt.so, or with trace=True the phase-stamping variant
    librgt_trace.so (same ABI; the fused kernel writes per-workgroup clock
    stamps after the regular workspace regions)."""
    lib = TRACE_LIB if trace else LIB
    us = units(trace)
    os.makedirs(os.path.dirname(us[0][1]), exist_ok=True)
    cc = hipcc()
    cmds = [[cc, *compile_flags(), *extra, "-c", src, "-o", obj] for src, obj, extra in us]
    jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = lib + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-fPIC", "-shared", *[o for _, o, _ in us],
          "-Wl,-rpath,/opt/rocm/lib", "-o", tmp], verbose)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True, trace="--trace" in sys.argv))
