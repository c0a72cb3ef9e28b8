"""Build libtide.so (C ABI + gfx950 kernels) and libtide_probe.so in-tree with hipcc.

    python -m all_gather_placement_amd.build

The libraries are compiled for gfx950 only.  Packed-fp32 instructions are disabled for device code
(the kernels' fp32 adds must stay plain IEEE adds in a fixed order), and no fast-math flag is
used, so fp32 denormals and rounding are IEEE.

Each library embeds a build id: the first 16 hex digits of the SHA-256 of its sources, the headers
they include and the compile flags (``tide_build_id()`` / ``tide_probe_build_id()``).
:func:`ensure_built` rebuilds a library whose embedded id differs from the sources in the tree, and
the bindings refuse to load one, so a library built from other sources is never run.
"""
from __future__ import annotations

import ctypes
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtide.so")
SOURCES = ["layout.cpp", "api.cpp", "kernels.hip"]
PROBE_LIB = os.path.join(PKG, "libtide_probe.so")
PROBE_SOURCES = ["probe.hip"]
ARCH = "gfx950"

# Everything each library is compiled from (its sources and every header they include).
HASHED = {
    LIB: [os.path.join(CSRC, f) for f in ("layout.cpp", "api.cpp", "kernels.hip", "layout.h", "tide_internal.h")]
         + [os.path.join(INCLUDE, "tide.h")],
    PROBE_LIB: [os.path.join(CSRC, f) for f in ("probe.hip", "tide_internal.h")]
               + [os.path.join(INCLUDE, "tide_probe.h")],
}
ID_SYMBOL = {LIB: "tide_build_id", PROBE_LIB: "tide_probe_build_id"}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (looked in $HIPCC, /opt/rocm/bin, PATH)")


def compile_flags(extra=()) -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, *extra,
    ]


def source_hash(lib: str = LIB, extra=()) -> str:
    """Build id of `lib` for the sources now in the tree (16 hex digits)."""
    h = hashlib.sha256()
    for path in HASHED[lib]:
        h.update(os.path.basename(path).encode() + b"\0")
        with open(path, "rb") as fh:
            h.update(fh.read())
        h.update(b"\0")
    h.update(" ".join(compile_flags(extra)).replace(INCLUDE, "<include>").encode())
    return h.hexdigest()[:16]


def built_id(lib: str = LIB):
    """Build id embedded in the library file at `lib`, or None if it is missing or carries none.
    Loads the library (no HIP call is made by loading or by the id query)."""
    if not os.path.exists(lib):
        return None
    try:
        fn = getattr(ctypes.CDLL(lib), ID_SYMBOL[lib])
    except (OSError, AttributeError):
        return None
    fn.restype = ctypes.c_char_p
    fn.argtypes = []
    return fn().decode()


def check_current(lib: str = LIB, loaded=None) -> None:
    """Raise if the library (the file, or the already loaded CDLL `loaded`) was not built from the
    sources now in the tree."""
    want = source_hash(lib)
    if loaded is not None:
        fn = getattr(loaded, ID_SYMBOL[lib], None)
        got = None
        if fn is not None:
            fn.restype = ctypes.c_char_p
            fn.argtypes = []
            got = fn().decode()
    else:
        got = built_id(lib)
    if got != want:
        raise RuntimeError(f"{lib} was built from other sources (build id {got}, sources {want}); "
                           f"rebuild it: python -m all_gather_placement_amd.build")


def build(verbose: bool = False, extra=(), out: str = LIB, sources=SOURCES, probe: bool = True) -> str:
    """Compile every source and link the shared library (and the probe library); returns its path."""
    if probe and out == LIB:
        build(verbose=verbose, extra=extra, out=PROBE_LIB, sources=PROBE_SOURCES, probe=False)
    objdir = os.path.join(PKG, "_build", os.path.splitext(os.path.basename(out))[0])
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    key = out if out in HASHED else LIB
    bid = source_hash(key, extra)
    id_flag = [f"-DTIDE_BUILD_ID=\"{bid}\""]
    objs = []
    for src in sources:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, *compile_flags(extra), *id_flag, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = out + ".tmp"
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp,
            "-Wl,-rpath,/opt/rocm/lib", "-L/opt/rocm/lib", "-lamdhip64"]
    if out == PROBE_LIB:
        link.append("-lhsa-runtime64")  # the DMA engines' rectangular copy (tide_probe_dma_rect_copies)
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, out)
    return out


def is_current(lib: str) -> bool:
    """True when `lib` exists and carries the build id of the sources now in the tree.  The id is
    read in a child process, so a stale file is never mapped into this one (it may be rebuilt)."""
    if not os.path.exists(lib):
        return False
    code = ("import sys; sys.path.insert(0, %r); from all_gather_placement_amd.build import built_id; "
            "print(built_id(%r) or '')" % (ROOT, lib))
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True)
    return res.returncode == 0 and res.stdout.strip() == source_hash(lib)


def ensure_built(verbose: bool = False) -> str:
    """Build the libraries if they are missing or were built from other sources (tests, smoke and
    benchmark entry points); returns the path of libtide.so."""
    if not (is_current(LIB) and is_current(PROBE_LIB)):
        build(verbose=verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
