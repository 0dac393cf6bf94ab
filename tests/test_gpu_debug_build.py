"""The debug build of the library (KVSEL_DEBUG=1, libkvsel_debug.so): its
kernels count every failed device-side check (a K/V row outside its pool, an
LDS index outside its array, an output slot outside its row, a split counter
that did not start at zero, a count past its bound) instead of trapping.

  * the GPU kernel tests, the workload tests at reduced sizes and the full
    C2, N1-profiling and draft-verification runs pass against it, each test
    ending with no failed check (the autouse fixture in conftest.py);
  * a workspace whose split counter was left non-zero -- a caller's misuse the
    release build cannot see -- is reported with the counter's value.

Both run in a child process that loads the debug build."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEBUG_LIB = os.path.join(ROOT, "decode_focal_layer_amd", "libkvsel_debug.so")
pytestmark = pytest.mark.gpu


def _env():
    if not os.path.exists(DEBUG_LIB):
        raise RuntimeError(f"{DEBUG_LIB} is not built (python -m decode_focal_layer_amd.build --debug)")
    return dict(os.environ, KVSEL_LIBRARY=DEBUG_LIB, PYTHONUNBUFFERED="1")


def test_kernel_tests_pass_every_device_check():
    print("[case] kernel and workload tests against the debug build", flush=True)
    r = subprocess.run([sys.executable, "-u", "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "gpu",
                        "tests/test_gpu_kernels.py", "tests/test_gpu_configs.py", "tests/test_gpu_full.py"],
                       cwd=ROOT, env=_env(), capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and " passed" in out, out[-4000:]
    print(out.strip().splitlines()[-1], flush=True)


STALE_COUNTER = r"""
import numpy as np, torch
from decode_focal_layer_amd import kvsel
from tests.gpu_util import random_paged
assert kvsel.LIB_PATH.endswith("libkvsel_debug.so")
rng = np.random.default_rng(5)
batch, hkv, G, n = 2, 2, 2, 3000                  # few pairs: each pair's rows split over work-groups
kp, vp, table = random_paged(rng, batch, hkv, n, "cuda")
i32 = lambda x: torch.tensor(x, dtype=torch.int32, device="cuda")
kv = kvsel.KV(kp, vp, torch.from_numpy(table).cuda(), i32([n, n]), i32([0, 0]), i32([2000, 2000]),
              max_seq_len=n, max_seg_len=2000, min_seg_len=2000)
q = torch.randn((batch, hkv * G, 128), device="cuda").to(torch.bfloat16)
idx = torch.from_numpy(np.sort(rng.choice(2000, size=(batch, hkv, 100)), axis=-1).astype(np.int32)).cuda()
out = torch.zeros((batch, hkv * G, 128), dtype=torch.float32, device="cuda")
ws = kvsel.Workspace("cuda")
kvsel.gather_attn(kv, q, hkv * G, 0.088, idx, 100, out, ws=ws)
torch.cuda.synchronize()
clean = kvsel.debug_status()
p, _ = ws.ptr_and_size(0)
off = p.value - ws.buf.data_ptr()
ws.buf[off:off + 4] = torch.tensor([7, 0, 0, 0], dtype=torch.uint8, device="cuda")   # pair (0, 0)'s counter: 7
kvsel.gather_attn(kv, q, hkv * G, 0.088, idx, 100, out, ws=ws)
torch.cuda.synchronize()
stale = kvsel.debug_status()
ws.buf.zero_()
torch.cuda.synchronize()
print("RESULT", *clean, *stale)
"""


def test_stale_split_counter_is_reported():
    print("[case] a split counter left at 7 in the workspace, debug build", flush=True)
    r = subprocess.run([sys.executable, "-c", STALE_COUNTER], cwd=ROOT, env=_env(), capture_output=True, text=True,
                       timeout=300)
    out = r.stdout + r.stderr
    line = [l for l in r.stdout.splitlines() if l.startswith("RESULT")]
    assert r.returncode == 0 and line, out[-4000:]
    v = [int(x) for x in line[0].split()[1:]]
    assert v[:4] == [0, 0, 0, 0], f"clean call: {v[:4]}"
    st, nviol, code, detail = v[4:]
    # every work-group of that pair arrives at 7, 8, ...; the first failed check recorded is one of them
    assert st == -5 and nviol >= 1 and code == 4 and 7 <= detail < 7 + 64, f"stale counter: {v[4:]}"
