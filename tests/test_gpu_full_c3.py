"""Full-size parity of FastKV-style decode under a compressed KV budget
(batch 16, 8 kv / 32 q heads, 131072-token source context, 8 physical
caches aliased by 32 logical layers, 2048 kept rows per kv head + the 64
recent rows + the rows generated since, 128 steps), run once through the
drivers the benchmark times.

Checked against the oracle:
  * every selection: all 8 caches x 16 sequences x 8 kv heads (1024 rows of
    131008 candidates: window scores of the last 8 queries, causal, context
    normalised, summed over the group's heads and window rows, average pool
    of width 7, top-2048), by the tie-band rule;
  * every one of the 128 steps of logical layers 0, 1, 15 and 31, all 128
    (sequence, kv head) pairs, against the oracle's attention over the kept
    rows, the recent rows and the generated rows visible at that step.

FastKV (section 2A, Token-Selective Propagation: window saliency; section
2B, Decoupled KV Retention: the per-head budget).
"""
import types

import numpy as np
import pytest
import torch

import synth
from oracle import oracle as O
from synth import gen
from tests.gpu_util import BAND, assert_attn, keep_freed_memory, log_case, need_gpu, pair_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"
CHECK_LAYERS = (0, 1, 15, 31)


@pytest.fixture(scope="module")
def c3():
    need_gpu()
    keep_freed_memory()
    from decode_focal_layer_amd import kvsel
    from decode_focal_layer_amd.fastkv import BudgetDecoder
    cfg = synth.C3
    log_case("c3 full: generate")
    w = gen.make_budget(cfg, DEV)
    s0, s1 = cfg.seg
    kvs = [kvsel.KV(w.k_pool[p], w.v_pool[p], w.block_table, w.seq_len_sel, w.seg_begin, w.seg_end,
                    max_seq_len=cfg.src_len + cfg.steps, max_seg_len=s1 - s0, min_seg_len=s1 - s0)
           for p in range(cfg.phys_layers)]
    dec = BudgetDecoder(kvs, cfg.hq, cfg.k, cfg.layers, cfg.scale, cfg.window, cfg.pool, device=DEV)
    log_case("c3 full: select")
    for p in range(cfg.phys_layers):
        dec.select(p, w.qwin[p], w.seq_len_sel)
    sel = np.stack([dec.idx[p].cpu().numpy() for p in range(cfg.phys_layers)])    # [P, B, hkv, k]
    log_case("c3 full: decode 128 steps")
    outs = torch.empty((cfg.steps, len(CHECK_LAYERS), cfg.batch, cfg.hq, 128), dtype=torch.float32, device=DEV)
    for t in range(cfg.steps):
        dec.step(w.q[t], w.seq_len[t])
        outs[t].copy_(dec.out[list(CHECK_LAYERS)])
    torch.cuda.synchronize()
    ns = types.SimpleNamespace(cfg=cfg, w=w, sel=sel, outs=outs.cpu().numpy(), qwin=w.qwin.cpu(),
                               q=w.q[:, list(CHECK_LAYERS)].cpu())
    yield ns
    del dec, kvs, ns.w, w, outs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("p", range(8))
def test_c3_selection(c3, p):
    """Physical cache p: the kept set of every (sequence, kv head)."""
    cfg, w = c3.cfg, c3.w
    s0, s1 = cfg.seg
    G = cfg.group
    log_case("c3 selection, cache", p)
    bad = []
    for b in range(cfg.batch):
        for g in range(cfg.hkv):
            Kl = O.logical_rows(w.k_pool[p], w.table_np[b], g, cfg.src_len)
            qw = O.widen(c3.qwin[p, b, :, g * G:(g + 1) * G])                        # [W, G, d]
            ref = O.avg_pool(O.window_scores(qw, Kl, s0, s1, cfg.scale, cfg.causal), cfg.pool)
            ok, nd = O.tie_band_check(c3.sel[p, b, g], ref, cfg.k, BAND)
            if not ok:
                bad.append((b, g, nd))
    assert not bad, f"cache {p}: kept sets outside the tie band (seq, kv head, n_diff): {bad[:10]}"


@pytest.mark.parametrize("li", range(len(CHECK_LAYERS)))
def test_c3_every_step(c3, li):
    """Logical layer CHECK_LAYERS[li] at every step, every pair.  The rows a
    pair may attend over the whole run (its kept rows, the recent rows, every
    appended row) are read once; step t's query sees those at positions up
    to src_len + t."""
    cfg, w = c3.cfg, c3.w
    l = CHECK_LAYERS[li]
    p = l % cfg.phys_layers
    s0, s1 = cfg.seg
    G, T = cfg.group, cfg.steps
    n_end = cfg.src_len + T
    log_case("c3 every step, layer", l)
    for b in range(cfg.batch):
        for g in range(cfg.hkv):
            rows = np.sort(O.kept_rows(c3.sel[p, b, g], s0, s1, n_end))
            Kr = pair_rows(w.k_pool[p], w.table_np[b], g, rows)
            Vr = pair_rows(w.v_pool[p], w.table_np[b], g, rows)
            vis = rows[None, None, :] < (cfg.src_len + 1 + np.arange(T))[:, None, None]   # [T, 1, rows]
            qg = O.widen(c3.q[:, li, b, g * G:(g + 1) * G])                          # [T, G, d]
            ref, _ = O.attention_masked(qg, Kr, Vr, vis, cfg.scale)
            for t in range(T):
                assert_attn(c3.outs[t, li, b, g * G:(g + 1) * G], ref[t], f"t{t} l{l} b{b} g{g}")
