"""A second build of libkvsel.so for host-side checking on the CPU: the same
sources and device code, the host code compiled with AddressSanitizer and
UndefinedBehaviorSanitizer (every sanitizer flag goes to the host pass only:
-Xarch_host).  The C-ABI's argument validators, the block pool and the fork
run on the host, so the CPU tests of the ABI and the pool exercise them
under the sanitizers by loading this library (KVSEL_LIBRARY) with the
sanitizer runtime preloaded.

Output: _build/host_sanitized/libkvsel.so, rebuilt only when a source, a
header or a flag changes (a hash of them is kept beside it).
"""
import glob
import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

from decode_focal_layer_amd import build as B

OUT = os.path.join(B.BUILD, "host_sanitized")
LIB = os.path.join(OUT, "libkvsel.so")
HOST_FLAGS = [f for pair in (("-Xarch_host", x) for x in (
    "-g", "-fno-omit-frame-pointer", "-fsanitize=address", "-fsanitize=undefined",
    "-fno-sanitize-recover=undefined")) for f in pair]
LINK_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan"]


def runtime() -> str:
    """The sanitizer runtime to preload (the compiler's own), or '' if absent."""
    clang_root = os.path.join(os.path.dirname(os.path.realpath(B.HIPCC)), "..", "lib", "llvm", "lib", "clang")
    found = sorted(glob.glob(os.path.join(clang_root, "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    return os.path.realpath(found[-1]) if found else ""


def _stamp() -> str:
    h = hashlib.sha256()
    for f in sorted(B.sources() + glob.glob(os.path.join(B.CSRC, "*.h")) +
                    glob.glob(os.path.join(B.ROOT, "include", "*.h"))):
        h.update(f.encode())
        h.update(open(f, "rb").read())
    h.update(" ".join(B.FLAGS + HOST_FLAGS + LINK_FLAGS).encode())
    return h.hexdigest()


def build(verbose: bool = False) -> str:
    os.makedirs(OUT, exist_ok=True)
    stamp_file = os.path.join(OUT, "stamp")
    stamp = _stamp()
    if os.path.exists(LIB) and os.path.exists(stamp_file) and open(stamp_file).read() == stamp:
        return LIB

    def one(src):
        obj = os.path.join(OUT, os.path.basename(src)[:-4] + ".o")
        r = subprocess.run([B.HIPCC, *B.FLAGS, *HOST_FLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(B.sources()))) as ex:
        objs = list(ex.map(one, B.sources()))
    r = subprocess.run([B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *LINK_FLAGS, *objs, "-o", LIB],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    for o in objs:
        os.remove(o)
    with open(stamp_file, "w") as f:
        f.write(stamp)
    if verbose:
        print(LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
