"""Build libkda.so (gfx950) in place with hipcc.

Used by ``__graft_entry__.build()``; run it directly with
``python -m linear_attention_sequence_kda_amd.build``.
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
LIB = os.path.join(PKG, "libkda.so")
SOURCES = ["kda_api.cpp", "kda_intra.hip", "kda_inter.hip", "kda_inter_scalar.hip", "kda_decode.hip",
           "kda_feature.hip", "kda_bwd.hip", "kda_scratch.hip",
           "kda_inter_wide.hip", "kda_chunk_bwd.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkda)")


def _flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            # packed fp32 VALU forms are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC]


def link_flags():
    """Libraries the ABI layer links: roctx of rocprofiler-sdk (one profiler
    range per ABI call)."""
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(hipcc())), "lib")
    return ["-L", rocm_lib, "-lrocprofiler-sdk-roctx", f"-Wl,-rpath,{rocm_lib}"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError("building libkda.so failed: " + " ".join(cmd[-3:]))


def build(verbose: bool = False) -> str:
    """Compile every source into libkda.so for gfx950 (always recompiles).

    Each source is compiled to an object of its own, in parallel, then the
    objects are linked into the shared library."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(ROOT, "_build", "obj")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    jobs = [[hipcc()] + _flags() + ["-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max(1, min(len(jobs), os.cpu_count() or 1))) as ex:
        for f in [ex.submit(_run, j, verbose) for j in jobs]:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + link_flags() + ["-o", tmp],
         verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
