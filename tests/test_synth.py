"""Harness self-checks: seeded inputs are reproducible and have the stated
structure (no arithmetic of the method is involved)."""
import numpy as np
import torch

import synth
from synth import gen


def test_seeds_reproducible_and_distinct():
    a = gen.normal_bf16((4, 8), ("x", 1), "cpu")
    b = gen.normal_bf16((4, 8), ("x", 1), "cpu")
    c = gen.normal_bf16((4, 8), ("x", 2), "cpu")
    assert torch.equal(a, b) and not torch.equal(a, c)
    assert a.dtype == torch.bfloat16


def test_raster_walk_wraps():
    walk = gen.raster_walk(8, 20, 4, 16, 6, (0, 0), [2, 2, 2, 2, 2, 2])
    assert walk[:3] == [(0, 0), (0, 2), (0, 4)]
    assert walk[3] == (4, 0)                  # 6 + 16 > 20 -> next patch row
    walk = gen.raster_walk(8, 20, 4, 16, 4, (4, 4), [1, 1, 1, 1])
    assert walk[1] == (0, 0)                  # bottom reached -> back to row 0
    for r, c in gen.raster_walk(80, 80, 4, 16, 200, (3, 5), np.random.default_rng(0).integers(1, 3, 200)):
        assert 0 <= r <= 76 and 0 <= c <= 64


def test_focal_small_structure():
    cfg = synth.small(synth.C4, batch=5, layers=2, steps=3, focal=(1,), grid_rows=8, grid_cols=16,
                      n_always=16, suffix_range=(3, 40))
    w = gen.make_focal(cfg, "cpu")
    assert np.all((w.suffix_len >= 3) & (w.suffix_len <= 40))
    pref = cfg.prefix_len // cfg.block
    assert np.all(w.table_np[:, :pref] == np.arange(pref)[None, :])
    own = [set(w.table_np[b, pref:pref + (-(-(int(w.suffix_len[b]) + 3) // 16))].tolist()) for b in range(5)]
    for i in range(5):
        for j in range(i + 1, 5):
            assert not (own[i] & own[j])
    assert w.seq_len_np[2, 0] == cfg.prefix_len + w.suffix_len[0] + 3
    w2 = gen.make_focal(cfg, "cpu")
    assert torch.equal(w.q, w2.q) and torch.equal(w.k_pool[1], w2.k_pool[1])


def test_key_side_patch_moves_keys_toward_query():
    cfg = synth.small(synth.C0, grid_rows=8, grid_cols=32, n_always=32)
    w = gen.make_focal(cfg, "cpu")
    r, c = w.patches[0, 0]
    toks = gen.patch_tokens(int(r), int(c), cfg.grid_cols, 4, 16)
    K = w.k_pool[0].float().permute(0, 2, 1, 3).reshape(-1, cfg.hkv, 128)   # contiguous table, b = 0
    q = w.q[0, 0, 0].float().view(cfg.hkv, 2, 128).sum(1)
    qhat = q / q.norm(dim=-1, keepdim=True)
    proj = (K * qhat[None]).sum(-1)                               # [N, hkv]
    inside = proj[torch.from_numpy(toks)].mean()
    mask = torch.ones(K.shape[0], dtype=torch.bool)
    mask[torch.from_numpy(toks)] = False
    assert inside - proj[mask].mean() > 0.3


def test_budget_rounding():
    assert synth.budget(0.05, 3584) == 179
    assert synth.budget(0.2, 32768) == 6554
    assert synth.budget(0.05, 3072) == 154
    assert synth.budget(0.05, 6400) == 320
