"""Full-size parity of the HPD-style branched decode: 512 branches over one
shared prefix of 4096 rows (3072 visual in a 48 x 64 grid, then 1024
layout rows) referenced zero-copy through every branch's block table, a
private suffix of U[32, 1024] rows per branch, 28 layers, focal layers 3
and 14 keeping the top 154 visual rows, 32 steps.  Both forms are run: each
branch attending over its own rows directly, and the cascade the benchmark
times (the shared layout rows, or for the focal layers the whole prefix
with its segment logits, once per kv head for all branches, merged exactly
with each branch's own rows; the focal selection from those logits).

Checked against the oracle, in both forms:
  * all 512 x 8 kept sets of both focal layers at steps 0, 1 and 31, by the
    tie-band rule;
  * all 28 layers' outputs of 48 (branch, kv head) pairs -- every kv head
    appears -- at steps 0, 1 and 31.

HPD-Parsing wiki, method item 2 (shared-prefix KV reuse); FastOCR
(Focal-Guided Pruning, Cross-Layer Propagation, Cross-Step Fixation Reuse).
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
CHECK_STEPS = (0, 1, 31)
FORMS = ("direct", "cascade")


@pytest.fixture(scope="module")
def c4():
    need_gpu()
    keep_freed_memory()
    from decode_focal_layer_amd import kvsel
    from decode_focal_layer_amd.decode import FocalDecoder
    cfg = synth.C4
    log_case("c4 full: generate")
    w = gen.make_focal(cfg, DEV)
    max_len = int(w.seq_len_np.max())
    kvs = [kvsel.KV(w.k_pool[l], w.v_pool[l], w.block_table, w.seq_len[0], w.seg_begin, w.seg_end,
                    max_seq_len=max_len, max_seg_len=cfg.n_visual, min_seg_len=cfg.n_visual,
                    shared_rows=cfg.prefix_len)
           for l in range(cfg.layers)]
    need_sets = sorted(set(CHECK_STEPS) | {t - 1 for t in CHECK_STEPS if t > 0})
    res = {}
    for form in FORMS:
        log_case("c4 full: decode 32 steps,", form)
        dec = FocalDecoder(kvs, cfg.hq, cfg.k, cfg.focal, cfg.scale, cfg.n_visual, device=DEV,
                           shared_tail=(cfg.n_visual, cfg.prefix_len) if form == "cascade" else None)
        sets, outs = {}, {}
        for t in range(cfg.steps):
            dec.step(t, w.q[t], w.seq_len[t])
            if t in need_sets:
                sets[t] = torch.stack([dec.selection(f).clone() for f in cfg.focal])
            if t in CHECK_STEPS:
                outs[t] = dec.out.clone()
        torch.cuda.synchronize()
        res[form] = ({t: s.cpu().numpy() for t, s in sets.items()}, {t: o.cpu().numpy() for t, o in outs.items()})
        del dec
    # the shared prefix is the same blocks in every branch's table
    pb = cfg.prefix_len // cfg.block
    assert np.all(w.table_np[:, :pb] == w.table_np[0, :pb])
    ns = types.SimpleNamespace(cfg=cfg, w=w, res=res, q=w.q[list(CHECK_STEPS)].cpu())
    yield ns
    del kvs, ns.w, w
    torch.cuda.empty_cache()


@pytest.mark.parametrize("form", FORMS)
def test_c4_kept_sets(c4, form):
    """Every (branch, kv head) kept set of both focal layers at the checked
    steps.  The visual segment is the shared prefix, the same rows for every
    branch (read once through branch 0's table)."""
    cfg, w = c4.cfg, c4.w
    sets, _ = c4.res[form]
    G = cfg.group
    bad = []
    for fi, f in enumerate(cfg.focal):
        log_case("c4 kept sets,", form, "layer", f)
        for g in range(cfg.hkv):
            Kseg = O.logical_rows(w.k_pool[f], w.table_np[0], g, cfg.n_visual)
            for i, t in enumerate(CHECK_STEPS):
                qg = O.widen(c4.q[i, f, :, g * G:(g + 1) * G])                       # [branches, G, d]
                s = O.focal_scores(qg, Kseg, 0, cfg.n_visual, cfg.scale)              # [branches, n_visual]
                ok, nd = O.tie_band_check(sets[t][fi, :, g], s, cfg.k, BAND)
                bad += [(t, f, b, g, int(nd[b])) for b in np.nonzero(~ok)[0]]
    assert not bad, f"{form}: kept sets outside the tie band (step, layer, branch, kv head, n_diff): {bad[:10]}"


def _out_pairs(cfg):
    """48 pairs spread over the branches, kv head = branch index mod 8."""
    bs = np.linspace(0, cfg.batch - 1, 48).round().astype(int)
    return [(int(b), int(b) % cfg.hkv) for b in bs]


@pytest.mark.parametrize("form", FORMS)
def test_c4_outputs(c4, form):
    """All 28 layers' outputs of 48 pairs at the checked steps."""
    cfg, w = c4.cfg, c4.w
    sets, outs = c4.res[form]
    G, T = cfg.group, len(CHECK_STEPS)
    plans = {t: O.focal_layer_plan(cfg.layers, cfg.focal, t) for t in CHECK_STEPS}
    for l in range(cfg.layers):
        log_case("c4 outputs,", form, "layer", l)
        for b, g in _out_pairs(cfg):
            n_t = [int(w.seq_len_np[t, b]) for t in CHECK_STEPS]
            n_max = max(n_t)
            pos = np.arange(n_max)
            Kl = O.logical_rows(w.k_pool[l], w.table_np[b], g, n_max)
            Vl = O.logical_rows(w.v_pool[l], w.table_np[b], g, n_max)
            vis = np.zeros((T, 1, n_max), dtype=bool)
            for i, t in enumerate(CHECK_STEPS):
                e = plans[t][l]
                if e[0] in ("dense", "focal"):
                    vis[i, 0] = pos < n_t[i]
                else:
                    src = sets[e[2]][cfg.focal.index(e[3]), b, g]
                    vis[i, 0, O.kept_rows(src, 0, cfg.n_visual, n_t[i])] = True
            qg = O.widen(c4.q[:, l, b, g * G:(g + 1) * G])                            # [T, G, d]
            ref, _ = O.attention_masked(qg, Kl, Vl, vis, cfg.scale)
            for i, t in enumerate(CHECK_STEPS):
                assert_attn(outs[t][l, b, g * G:(g + 1) * G], ref[i], f"{form} t{t} l{l} {plans[t][l][0]} b{b} g{g}")
