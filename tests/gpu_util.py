"""Shared helpers of the GPU parity tests: build descriptors from synthetic
workloads, pull logical rows for the oracle, and the acceptance checks."""
import math

import numpy as np
import pytest
import torch

from oracle import oracle as O

ATOL = 2e-3      # attention: max abs error
RTOL_L2 = 1e-3   # attention: relative L2 error
BAND = 1e-6      # kept sets: relative tie band around the k-th score


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_focal_layer_amd import kvsel
    kvsel.lib()   # fails loudly when the library is missing


def attn_errors(gpu, ref):
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    max_abs = float(np.abs(g - r).max()) if g.size else 0.0
    l2 = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))
    return max_abs, l2


def assert_attn(gpu, ref, what=""):
    max_abs, l2 = attn_errors(gpu, ref)
    assert max_abs <= ATOL and l2 <= RTOL_L2, f"{what}: max_abs={max_abs:.3e} relL2={l2:.3e}"
    return max_abs, l2


def rel_err(gpu, ref):
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    return float((np.abs(g - r) / np.maximum(np.abs(r), 1e-30)).max())


def random_paged(rng, batch, hkv, max_len, device, extra_blocks=3):
    """A bf16 pool with a random block permutation and its block table."""
    mb = -(-max_len // 16)
    nb = batch * mb + extra_blocks
    perm = rng.permutation(nb)[: batch * mb].reshape(batch, mb).astype(np.int32)
    g = torch.Generator().manual_seed(int(rng.integers(1 << 30)))
    k = torch.randn((nb, hkv, 16, 128), generator=g).to(torch.bfloat16).to(device)
    v = torch.randn((nb, hkv, 16, 128), generator=g).to(torch.bfloat16).to(device)
    return k, v, perm


def cpu_pool(t):
    return t.detach().cpu()


def log_case(*parts):
    print("[case]", *parts, flush=True)


def keep_freed_memory():
    """Let the C heap keep freed blocks of any size instead of returning them
    to the system, so the full-size checks, which allocate and free arrays
    of tens of MB per (sequence, kv head), do not page-fault them in again
    each time (mallopt M_MMAP_THRESHOLD and M_TRIM_THRESHOLD)."""
    import ctypes
    try:
        libc = ctypes.CDLL("libc.so.6")
    except OSError:
        return
    libc.mallopt(-3, 1 << 30)   # M_MMAP_THRESHOLD
    libc.mallopt(-1, 1 << 30)   # M_TRIM_THRESHOLD


def pair_rows(pool, table_row, g, rows):
    """K or V rows at logical positions `rows` of one sequence's kv head g,
    float64 on the host: the paged read (block table_row[j // 16], offset
    j % 16) applied to a subset of positions."""
    rows = np.asarray(rows, dtype=np.int64)
    blk = torch.from_numpy(np.asarray(table_row, dtype=np.int64)[rows // 16]).to(pool.device)
    off = torch.from_numpy(rows % 16).to(pool.device)
    return O.widen(pool[blk, g, off, :])
