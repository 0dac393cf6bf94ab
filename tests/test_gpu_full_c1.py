"""Full-size parity of the FastOCR-style decode (batch 32, 28 layers, 64
steps, 6400 visual + 1024 text rows, focal layers 3 and 14, warm-started
top-320), run once through the decoder the benchmark times.

Checked against the oracle:
  * every kept set of both focal layers at every one of the 64 steps, all
    32 x 8 (sequence, kv head) pairs, by the tie-band rule;
  * every output: all 28 layers, all 32 x 8 (sequence, kv head) pairs, all
    64 steps, each layer against the oracle's attention over the rows the
    schedule gives it (dense, the same step's focal set, or the deepest focal
    set of the previous step), the sets being the validated GPU ones.

FastOCR (technical summary, Focal-Guided Pruning, Cross-Layer Propagation,
Cross-Step Fixation Reuse).
"""
import types

import numpy as np
import pytest
import torch

import synth
from oracle import oracle as O
from synth import gen
from tests.gpu_util import BAND, assert_attn, keep_freed_memory, log_case, need_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def c1():
    need_gpu()
    keep_freed_memory()
    from decode_focal_layer_amd import kvsel
    from decode_focal_layer_amd.decode import FocalDecoder
    cfg = synth.C1
    log_case("c1 full: generate")
    w = gen.make_focal(cfg, DEV)
    max_len = int(w.seq_len_np.max())
    kvs = [kvsel.KV(w.k_pool[l], w.v_pool[l], w.block_table, w.seq_len[0], w.seg_begin, w.seg_end,
                    max_seq_len=max_len, max_seg_len=cfg.n_visual, min_seg_len=cfg.n_visual)
           for l in range(cfg.layers)]
    dec = FocalDecoder(kvs, cfg.hq, cfg.k, cfg.focal, cfg.scale, cfg.n_visual, device=DEV)
    sets = torch.empty((cfg.steps, len(cfg.focal), cfg.batch, cfg.hkv, cfg.k), dtype=torch.int32, device=DEV)
    outs = torch.empty((cfg.steps,) + tuple(dec.out.shape), dtype=torch.float32, device=DEV)
    log_case("c1 full: decode 64 steps")
    for t in range(cfg.steps):
        dec.step(t, w.q[t], w.seq_len[t])
        for i, f in enumerate(cfg.focal):
            sets[t, i].copy_(dec.selection(f))
        outs[t].copy_(dec.out)
    torch.cuda.synchronize()
    ns = types.SimpleNamespace(cfg=cfg, w=w, sets=sets.cpu().numpy(), outs=outs.cpu().numpy(), q=w.q.cpu())
    yield ns
    del dec, kvs, ns.w, w
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fi", [0, 1])
def test_c1_kept_sets_every_step(c1, fi):
    """Focal layer cfg.focal[fi]: its kept set of every (sequence, kv head)
    at every step, against the oracle's segment-normalised group scores."""
    cfg, w = c1.cfg, c1.w
    f = cfg.focal[fi]
    G = cfg.group
    log_case("c1 kept sets, layer", f)
    bad = []
    for b in range(cfg.batch):
        for g in range(cfg.hkv):
            Kseg = O.logical_rows(w.k_pool[f], w.table_np[b], g, cfg.n_visual)    # the segment's rows
            qg = O.widen(c1.q[:, f, b, g * G:(g + 1) * G])                       # [steps, G, d]
            s = O.focal_scores(qg, Kseg, 0, cfg.n_visual, cfg.scale)              # [steps, n_visual]
            ok, nd = O.tie_band_check(c1.sets[:, fi, b, g], s, cfg.k, BAND)
            bad += [(t, b, g, int(nd[t])) for t in np.nonzero(~ok)[0]]
    assert not bad, f"layer {f}: kept sets outside the tie band (step, seq, kv head, n_diff): {bad[:10]}"


@pytest.mark.parametrize("quarter", range(4))
def test_c1_outputs(c1, quarter):
    """Every output of layers 7q .. 7q+6: all pairs, all steps."""
    cfg, w = c1.cfg, c1.w
    G, T = cfg.group, cfg.steps
    layers = range(7 * quarter, cfg.layers if quarter == 3 else min(7 * quarter + 7, cfg.layers))
    n_t = w.seq_len_np[:, 0].astype(np.int64)
    assert np.all(w.seq_len_np == n_t[:, None])
    n_max = int(n_t.max())
    plans = [O.focal_layer_plan(cfg.layers, cfg.focal, t) for t in range(T)]
    pos = np.arange(n_max)
    dense_vis = pos[None, :] < n_t[:, None]                                    # [T, n_max]
    for l in layers:
        log_case("c1 outputs, layer", l)
        for b in range(cfg.batch):
            for g in range(cfg.hkv):
                Kl = O.logical_rows(w.k_pool[l], w.table_np[b], g, n_max)
                Vl = O.logical_rows(w.v_pool[l], w.table_np[b], g, n_max)
                vis = np.zeros((T, 1, n_max), dtype=bool)
                for t in range(T):
                    e = plans[t][l]
                    if e[0] in ("dense", "focal"):
                        vis[t, 0] = dense_vis[t]
                    else:
                        src = c1.sets[e[2], cfg.focal.index(e[3]), b, g]
                        vis[t, 0, O.kept_rows(src, 0, cfg.n_visual, int(n_t[t]))] = True
                qg = O.widen(c1.q[:, l, b, g * G:(g + 1) * G])                  # [T, G, d]
                ref, _ = O.attention_masked(qg, Kl, Vl, vis, cfg.scale)
                for t in range(T):
                    assert_attn(c1.outs[t, l, b, g * G:(g + 1) * G], ref[t], f"t{t} l{l} {plans[t][l][0]} b{b} g{g}")
