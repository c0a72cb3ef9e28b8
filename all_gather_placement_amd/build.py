"""Build libtide.so (C ABI + gfx950 kernels) in-tree with hipcc.

    python -m all_gather_placement_amd.build

The library is compiled for gfx950 only.  Packed-fp32 instructions are disabled for device code
(the kernels' fp32 adds must stay plain IEEE adds in a fixed order), and no fast-math flag is
used, so fp32 denormals and rounding are IEEE.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libtide.so")
SOURCES = ["layout.cpp", "api.cpp", "kernels.hip"]
PROBE_LIB = os.path.join(PKG, "libtide_probe.so")
PROBE_SOURCES = ["probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (looked in $HIPCC, /opt/rocm/bin, PATH)")


def compile_flags(extra=()) -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), *extra,
    ]


def build(verbose: bool = False, extra=(), out: str = LIB, sources=SOURCES, probe: bool = True) -> str:
    """Compile every source and link the shared library (and the probe library); returns its path."""
    if probe and out == LIB:
        build(verbose=verbose, extra=extra, out=PROBE_LIB, sources=PROBE_SOURCES, probe=False)
    objdir = os.path.join(PKG, "_build", os.path.splitext(os.path.basename(out))[0])
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in sources:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, *compile_flags(extra), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = out + ".tmp"
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp,
            "-Wl,-rpath,/opt/rocm/lib", "-L/opt/rocm/lib", "-lamdhip64"]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, out)
    return out


def ensure_built(verbose: bool = False) -> str:
    """Build the libraries only if they are not there yet (tests, smoke and benchmark entry points);
    returns the path of libtide.so."""
    if not (os.path.exists(LIB) and os.path.exists(PROBE_LIB)):
        build(verbose=verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
