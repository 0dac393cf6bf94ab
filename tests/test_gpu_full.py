"""Full-size parity: the workloads at their stated sizes, in the launch
configuration the benchmark times, checked on sampled outputs that the
oracle computes one by one."""
import numpy as np
import pytest
import torch

import synth
from oracle import oracle as O
from synth import gen
from tests.gpu_util import BAND, assert_attn, log_case, need_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def test_c1_full_sampled():
    """C1 at full size (28 layers, batch 32, 64 steps) through the decoder the
    benchmark uses.  Checked: every kv head's kept set at both focal layers of
    steps 0, 1 and 63 (tie band); all 28 layers' outputs of 4 sampled
    (sequence, kv head) pairs at those steps."""
    from decode_focal_layer_amd import kvsel
    from decode_focal_layer_amd.decode import FocalDecoder
    cfg = synth.C1
    w = gen.make_focal(cfg, DEV)
    max_len = int(w.seq_len_np.max())
    kvs = [kvsel.KV(w.k_pool[l], w.v_pool[l], w.block_table, w.seq_len[0], w.seg_begin, w.seg_end,
                    max_seq_len=max_len, max_seg_len=cfg.n_visual, min_seg_len=cfg.n_visual)
           for l in range(cfg.layers)]
    dec = FocalDecoder(kvs, cfg.hq, cfg.k, cfg.focal, cfg.scale, cfg.n_visual, device=DEV)
    check_steps = {0, 1, cfg.steps - 1}
    rng = np.random.default_rng(5)
    pairs = [(int(rng.integers(cfg.batch)), int(rng.integers(cfg.hkv))) for _ in range(4)]
    sets, outs = {}, {}
    for t in range(cfg.steps):
        dec.step(t, w.q[t], w.seq_len[t])
        for f in cfg.focal:
            sets[(t, f)] = dec.selection(f).cpu().numpy() if (t in check_steps or t + 1 in check_steps) else None
        if t in check_steps:
            outs[t] = dec.out.cpu().numpy()
    torch.cuda.synchronize()
    G = cfg.group
    tables = w.table_np
    for t in sorted(check_steps):
        log_case("c1 full step", t)
        n = int(w.seq_len_np[t, 0])
        qc = w.q[t].cpu()
        plan = O.focal_layer_plan(cfg.layers, cfg.focal, t)
        # kept sets of every (sequence, kv head) at the focal layers
        for f in cfg.focal:
            kc = w.k_pool[f]
            for b in range(cfg.batch):
                for g in range(cfg.hkv):
                    Kl = O.logical_rows(kc, tables[b], g, n)
                    s = O.focal_scores(O.widen(qc[f, b, g * G:(g + 1) * G]), Kl, 0, cfg.n_visual, cfg.scale)
                    ok, nd = O.tie_band_check(sets[(t, f)][b, g], s, cfg.k, BAND)
                    assert ok, f"t{t} l{f} b{b} g{g}: {nd} indices differ outside the tie band"
        # every layer's output at sampled pairs
        for e in plan:
            l = e[1]
            for b, g in pairs:
                Kl = O.logical_rows(w.k_pool[l], tables[b], g, n)
                Vl = O.logical_rows(w.v_pool[l], tables[b], g, n)
                qg = O.widen(qc[l, b, g * G:(g + 1) * G])
                if e[0] in ("dense", "focal"):
                    ref, _ = O.dense_attention(qg, Kl, Vl, cfg.scale)
                else:
                    rows = O.kept_rows(sets[(e[2], e[3])][b, g], 0, cfg.n_visual, n)
                    ref, _ = O.attention(qg, Kl, Vl, rows, cfg.scale)
                assert_attn(outs[t][l, b, g * G:(g + 1) * G], ref, f"t{t} l{l} {e[0]} b{b} g{g}")


def test_c1_focal_layer_profiling():
    """Focal-layer choice on the C1 cache: 4 warm-up steps x 28 layers of
    image-attention ratios (batch 32, 16 heads), then the top-2 layers.
    Checked: 64 sampled (step, layer, sequence, kv head) ratios against the
    oracle, and the choice against the oracle's choice on the same ratios."""
    from decode_focal_layer_amd import kvsel
    from decode_focal_layer_amd.decode import FocalProfiler
    cfg = synth.C1
    w = gen.make_focal(cfg, DEV)
    max_len = int(w.seq_len_np.max())
    kvs = [kvsel.KV(w.k_pool[l], None, w.block_table, w.seq_len[0], w.seg_begin, w.seg_end,
                    max_seq_len=max_len, max_seg_len=cfg.n_visual, min_seg_len=cfg.n_visual)
           for l in range(cfg.layers)]
    W = 4
    prof = FocalProfiler(kvs, cfg.hq, cfg.scale, W, device=DEV)
    for t in range(W):
        prof.step(t, w.q[t], w.seq_len[t])
    layers = prof.pick(len(cfg.focal)).cpu().numpy()
    torch.cuda.synchronize()
    ratios = prof.ratios.cpu().numpy()
    assert np.array_equal(layers, O.pick_focal_layers(ratios.astype(np.float64), len(cfg.focal)))
    rng = np.random.default_rng(9)
    G, per = cfg.group, cfg.batch * cfg.hq
    for _ in range(64):
        t, l, b, g = (int(rng.integers(W)), int(rng.integers(cfg.layers)), int(rng.integers(cfg.batch)),
                      int(rng.integers(cfg.hkv)))
        n = int(w.seq_len_np[t, b])
        Kl = O.logical_rows(w.k_pool[l], w.table_np[b], g, n)
        ref = O.visual_mass(O.widen(w.q[t][l, b, g * G:(g + 1) * G].cpu()), Kl, 0, cfg.n_visual, cfg.scale)
        got = ratios[l, t * per + b * cfg.hq + g * G: t * per + b * cfg.hq + (g + 1) * G]
        assert np.abs(got - ref).max() <= 1e-5, (t, l, b, g)


def _rows(pool, table_row, g, rows):
    """K or V rows `rows` (logical positions) of one sequence's kv head g, as
    float64 on the host: the oracle's own paged-read applied to a subset."""
    rows = np.asarray(rows, dtype=np.int64)
    blk = torch.from_numpy(np.asarray(table_row, dtype=np.int64)[rows // 16]).to(pool.device)
    off = torch.from_numpy(rows % 16).to(pool.device)
    return O.widen(pool[blk, g, off, :])


def test_c2_full():
    """C2 in full: window scores summed over all 32 heads and pooled, top-6554,
    and the gather of the selected hidden rows plus the 8 window rows."""
    from decode_focal_layer_amd import kvsel
    from decode_focal_layer_amd.fastkv import tsp_select
    cfg = synth.C2
    w = gen.make_window(cfg, DEV)
    s0, s1 = cfg.seg
    kv = kvsel.KV(w.k_pool, None, w.block_table, w.seq_len, w.seg_begin, w.seg_end,
                  max_seq_len=cfg.prompt, max_seg_len=s1 - s0, min_seg_len=s1 - s0)
    log_case("c2 full")
    scores, idx, dst = tsp_select(kv, w.q, cfg.hq, cfg.scale, cfg.k, cfg.pool, hidden=w.hidden, window=cfg.window)
    torch.cuda.synchronize()
    G = cfg.group
    qc = w.q.cpu()
    total = np.zeros(s1 - s0)
    for g in range(cfg.hkv):
        Kl = O.logical_rows(w.k_pool, w.table_np[0], g, cfg.prompt)
        total += O.window_scores(O.widen(qc[0, :, g * G:(g + 1) * G]), Kl, s0, s1, cfg.scale, cfg.causal)
    ref = O.avg_pool(total, cfg.pool)
    got = scores[0, 0].cpu().numpy()
    rel = float((np.abs(got - ref) / np.abs(ref)).max())
    print("C2 max relative score error", rel)
    assert rel < 2e-6
    gi = idx[0].cpu().numpy()
    ok, nd = O.tie_band_check(gi, ref, cfg.k, BAND)
    assert ok, f"{nd} kept indices differ outside the tie band"
    hid = w.hidden.cpu().view(torch.int16).numpy()
    want = O.gather_rows(hid, gi, cfg.prompt - cfg.window, cfg.window)
    assert np.array_equal(dst.cpu().view(torch.int16).numpy(), want)
    print("salient positions among the kept:", len(np.intersect1d(gi, w.salient[0])), "of", cfg.n_salient)


def test_c3_full_sampled():
    """C3 at full size (16 x 131072 tokens, 8 physical caches, 32 layers, 128
    steps).  Checked: the kept sets of 16 sampled (sequence, kv head) pairs of
    two physical caches (tie band), and at steps 0, 63 and 127 every pair's
    output of logical layers 0, 1, 15 and 31."""
    from decode_focal_layer_amd import kvsel
    from decode_focal_layer_amd.fastkv import BudgetDecoder
    cfg = synth.C3
    w = gen.make_budget(cfg, DEV)
    s0, s1 = cfg.seg
    kvs = [kvsel.KV(w.k_pool[p], w.v_pool[p], w.block_table, w.seq_len_sel, w.seg_begin, w.seg_end,
                    max_seq_len=cfg.src_len + cfg.steps, max_seg_len=s1 - s0, min_seg_len=s1 - s0)
           for p in range(cfg.phys_layers)]
    dec = BudgetDecoder(kvs, cfg.hq, cfg.k, cfg.layers, cfg.scale, cfg.window, cfg.pool, device=DEV)
    log_case("c3 selection")
    sel = []
    for p in range(cfg.phys_layers):
        dec.select(p, w.qwin[p], w.seq_len_sel)
        sel.append(dec.idx[p].cpu().numpy())
    torch.cuda.synchronize()
    G = cfg.group
    rng = np.random.default_rng(9)
    for p in (0, cfg.phys_layers - 1):
        qw = w.qwin[p].cpu()
        for _ in range(8):
            b, g = int(rng.integers(cfg.batch)), int(rng.integers(cfg.hkv))
            Kl = O.logical_rows(w.k_pool[p], w.table_np[b], g, cfg.src_len)
            ref = O.avg_pool(O.window_scores(O.widen(qw[b, :, g * G:(g + 1) * G]), Kl, s0, s1, cfg.scale,
                                             cfg.causal), cfg.pool)
            ok, nd = O.tie_band_check(sel[p][b, g], ref, cfg.k, BAND)
            assert ok, f"p{p} b{b} g{g}: {nd} indices differ outside the tie band"
    check_steps, check_layers = {0, 63, cfg.steps - 1}, (0, 1, 15, cfg.layers - 1)
    outs = {}
    for t in range(cfg.steps):
        dec.step(w.q[t], w.seq_len[t])
        if t in check_steps:
            outs[t] = dec.out.cpu().numpy()
    torch.cuda.synchronize()
    for t in sorted(check_steps):
        log_case("c3 step", t)
        n = cfg.src_len + t + 1
        qc = w.q[t].cpu()
        for l in check_layers:
            p = l % cfg.phys_layers
            for b in range(cfg.batch):
                for g in range(cfg.hkv):
                    rows = O.kept_rows(sel[p][b, g], s0, s1, n)
                    Kr = _rows(w.k_pool[p], w.table_np[b], g, rows)
                    Vr = _rows(w.v_pool[p], w.table_np[b], g, rows)
                    ref, _ = O.attention(O.widen(qc[l, b, g * G:(g + 1) * G]), Kr, Vr, np.arange(len(rows)),
                                         cfg.scale)
                    assert_attn(outs[t][l, b, g * G:(g + 1) * G], ref, f"t{t} l{l} b{b} g{g}")


@pytest.mark.parametrize("cascade", [False, True])
def test_c4_full_sampled(cascade):
    """C4 at full size (512 branches over one shared 4096-token prefix, 28
    layers, 32 steps).  Checked at steps 0, 1 and 31: the kept sets of 64
    sampled (branch, kv head) pairs at both focal layers, and all 28 layers'
    outputs of 4 sampled pairs.  cascade: the configuration the benchmark
    times -- the shared layout rows (sparse layers) and the whole prefix with
    its logits (focal layers) once per kv head for all branches, merged with
    each branch's own rows, the focal selection from those logits."""
    from decode_focal_layer_amd import kvsel
    from decode_focal_layer_amd.decode import FocalDecoder
    cfg = synth.C4
    w = gen.make_focal(cfg, DEV)
    max_len = int(w.seq_len_np.max())
    kvs = [kvsel.KV(w.k_pool[l], w.v_pool[l], w.block_table, w.seq_len[0], w.seg_begin, w.seg_end,
                    max_seq_len=max_len, max_seg_len=cfg.n_visual, min_seg_len=cfg.n_visual,
                    shared_rows=cfg.prefix_len)
           for l in range(cfg.layers)]
    dec = FocalDecoder(kvs, cfg.hq, cfg.k, cfg.focal, cfg.scale, cfg.n_visual, device=DEV,
                       shared_tail=(cfg.n_visual, cfg.prefix_len) if cascade else None)
    check_steps = {0, 1, cfg.steps - 1}
    rng = np.random.default_rng(11)
    sel_pairs = [(int(rng.integers(cfg.batch)), int(rng.integers(cfg.hkv))) for _ in range(64)]
    out_pairs = sel_pairs[:4]
    sets, outs = {}, {}
    for t in range(cfg.steps):
        dec.step(t, w.q[t], w.seq_len[t])
        for f in cfg.focal:
            if t in check_steps or t + 1 in check_steps:
                sets[(t, f)] = dec.selection(f).cpu().numpy()
        if t in check_steps:
            outs[t] = dec.out.cpu().numpy()
    torch.cuda.synchronize()
    G = cfg.group
    for t in sorted(check_steps):
        log_case("c4 step", t)
        qc = w.q[t].cpu()
        for f in cfg.focal:
            for b, g in sel_pairs:
                n = int(w.seq_len_np[t, b])
                Kl = O.logical_rows(w.k_pool[f], w.table_np[b], g, n)
                s = O.focal_scores(O.widen(qc[f, b, g * G:(g + 1) * G]), Kl, 0, cfg.n_visual, cfg.scale)
                ok, nd = O.tie_band_check(sets[(t, f)][b, g], s, cfg.k, BAND)
                assert ok, f"t{t} l{f} b{b} g{g}: {nd} indices differ outside the tie band"
        for e in O.focal_layer_plan(cfg.layers, cfg.focal, t):
            l = e[1]
            for b, g in out_pairs:
                n = int(w.seq_len_np[t, b])
                Kl = O.logical_rows(w.k_pool[l], w.table_np[b], g, n)
                Vl = O.logical_rows(w.v_pool[l], w.table_np[b], g, n)
                qg = O.widen(qc[l, b, g * G:(g + 1) * G])
                if e[0] in ("dense", "focal"):
                    ref, _ = O.dense_attention(qg, Kl, Vl, cfg.scale)
                else:
                    ref, _ = O.attention(qg, Kl, Vl, O.kept_rows(sets[(e[2], e[3])][b, g], 0, cfg.n_visual, n),
                                         cfg.scale)
                assert_attn(outs[t][l, b, g * G:(g + 1) * G], ref, f"t{t} l{l} {e[0]} b{b} g{g}")


@pytest.mark.parametrize("cascade", [False, True, 3])
def test_c4_verify_full_sampled(cascade):
    """Draft verification at the benchmark's size: 512 branches over the C4
    cache (shared 3072 + 1024 prefix, suffix U[32,1024] + 32 appended rows),
    8 drafts, 154 kept visual rows per kv head, the launch the benchmark times
    (one layer here), directly and as the cascade (the shared layout rows
    once for all drafts).  Checked: 24 sampled (branch, kv head) pairs,
    every draft and head, against the oracle."""
    from decode_focal_layer_amd import kvsel
    cfg = synth.small(synth.C4, layers=1)
    m = 8
    w = gen.make_focal(cfg, DEV)
    T = cfg.steps
    seq = w.seq_len[T - 1]
    n_np = w.seq_len_np[T - 1].astype(np.int64)
    kv = kvsel.KV(w.k_pool[0], w.v_pool[0], w.block_table, seq, w.seg_begin, w.seg_end,
                  max_seq_len=int(n_np.max()), max_seg_len=cfg.n_visual, min_seg_len=cfg.n_visual,
                  shared_rows=cfg.prefix_len)
    g = torch.Generator(device=DEV).manual_seed(cfg.seed + 77)
    keys = torch.rand((cfg.batch * cfg.hkv, cfg.n_visual), generator=g, device=DEV)
    idx = keys.argsort(dim=1)[:, :cfg.k].sort(dim=1).values.to(torch.int32).view(cfg.batch, cfg.hkv, cfg.k)
    q = torch.randn((cfg.batch, m, cfg.hq, 128), generator=g, device=DEV).to(torch.bfloat16)
    out = torch.empty((cfg.batch, m, cfg.hq, 128), dtype=torch.float32, device=DEV)
    lse = torch.empty((cfg.batch, m, cfg.hq), dtype=torch.float32, device=DEV)
    log_case("c4-verify-full", cfg.batch, m, cascade)
    from decode_focal_layer_amd.decode import DraftVerifier
    # cascade: True folds the shared rows into the output in one part; 3 cuts
    # them into three parts merged with the own rows by kvsel_merge_attn
    ver = DraftVerifier(kv, m, cfg.hq, cfg.scale, shared_tail=(cfg.n_visual, cfg.prefix_len) if cascade else None,
                        shared_splits=3 if cascade == 3 else None, device=DEV)
    ver.verify(q, idx, cfg.k, out, lse)
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    G = cfg.group
    idx_c, q_c = idx.cpu().numpy(), q.cpu()
    for _ in range(24):
        b, h = int(rng.integers(cfg.batch)), int(rng.integers(cfg.hkv))
        n = int(n_np[b])
        Kl = O.logical_rows(w.k_pool[0], w.table_np[b], h, n)
        Vl = O.logical_rows(w.v_pool[0], w.table_np[b], h, n)
        rows = O.kept_rows(idx_c[b, h], 0, cfg.n_visual, n)
        ref, rl = O.verify_attention(O.widen(q_c[b, :, h * G:(h + 1) * G]), Kl, Vl, rows, n, cfg.scale)
        got = out[b, :, h * G:(h + 1) * G].cpu().numpy()
        assert_attn(got.reshape(-1, 128), ref.reshape(-1, 128), f"c4 verify b{b} g{h}")
        assert np.abs(lse[b, :, h * G:(h + 1) * G].cpu().numpy() - rl).max() < 1e-4
