"""The C-ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
the argument validators of every entry point and the block pool with its
fork, through the ABI and pool tests, run in a child process against the
sanitized build of the library (decode_focal_layer_amd.build_sanitized) with
the sanitizer runtime preloaded.  Any report fails the run (halt_on_error).
No GPU: the validators reject before any HIP call, and the pool is host
code."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_and_pool_under_host_sanitizers():
    from decode_focal_layer_amd import build_sanitized as S
    rt = S.runtime()
    if not rt:
        pytest.skip("the compiler's AddressSanitizer runtime is not installed")
    lib = S.build()
    env = dict(os.environ, LD_PRELOAD=rt, KVSEL_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",   # the interpreter's own allocations
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the build is instrumented (calls into both runtimes) ...
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle_" in syms
    # ... and a child with this environment maps it and the runtime
    probe = ("from decode_focal_layer_amd import kvsel; kvsel.lib(); "
             "maps = open('/proc/self/maps').read(); print(kvsel.LIB_PATH in maps, 'libclang_rt.asan' in maps)")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.stdout.split() == ["True", "True"], r.stdout + r.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_abi.py", "tests/test_pool.py"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0 and " passed" in out, out[-4000:]
