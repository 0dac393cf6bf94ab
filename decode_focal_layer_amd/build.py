"""Build libkvsel.so for gfx950 with hipcc, in-tree.

    python -m decode_focal_layer_amd.build [-v] [--debug]

Every HIP source under csrc/ is compiled to an object (in parallel) and the
objects are linked into decode_focal_layer_amd/libkvsel.so.  Always rebuilds.
With debug=True (--debug) the same sources are built with KVSEL_DEBUG=1 into
decode_focal_layer_amd/libkvsel_debug.so: the kernels then count failed
device-side checks (kvsel_debug_status); load it with KVSEL_LIBRARY.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvsel.so")
LIB_DEBUG = os.path.join(PKG, "libkvsel_debug.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-command-line-argument", "-fvisibility=hidden",
    # keep the compiler from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, verbose: bool, debug: bool = False) -> str:
    obj = os.path.join(BUILD, "debug" if debug else "", os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *FLAGS, *(["-DKVSEL_DEBUG=1"] if debug else []), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if verbose and out.strip():
        print(out)
    return obj


def build(verbose: bool = False, debug: bool = False) -> str:
    os.makedirs(os.path.join(BUILD, "debug") if debug else BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, debug), srcs))
    lib = LIB_DEBUG if debug else LIB
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, debug="--debug" in sys.argv))
