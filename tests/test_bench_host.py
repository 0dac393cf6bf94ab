"""The benchmark's host-side contract (no GPU): the multi-GPU refusal and the
algorithmic byte counts the roofline is computed from."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_c1_algorithmic_bytes():
    """Per layer at decode step t of C1 (32 sequences, 8 kv heads, 6400 visual
    + 1024 text rows, top-320): a dense or focal layer reads every K/V row once
    (32 x (7424 + t + 1) x 8 x 512 B); a sparse layer reads the 320 kept rows
    and every row outside the segment (32 x (1344 + t + 1) x 8 x 512 B); both
    also move the query, the fp32 output and (focal) the scores and indices."""
    import bench
    import synth
    cfg = synth.C1
    B, hkv, hq, d = 32, cfg.hkv, cfg.hq, cfg.head_dim
    for t in (0, 1, 63):
        dense, focal, sparse = bench.algorithmic_bytes(cfg, t, B)
        qo = B * hq * d * (2 + 4)
        idx = B * hkv * cfg.k * 4
        assert dense == B * hkv * (7424 + t + 1) * 512 + qo
        assert sparse == B * hkv * (1344 + t + 1) * 512 + qo + idx
        assert focal == dense + 2 * B * hkv * 6400 * 4 + idx
    # the 64-step mean of a whole step is 6.68 GB without the small terms
    mean = sum(bench.step_bytes(cfg, t, B) for t in range(64)) / 64
    assert 6.68e9 < mean < 6.80e9
