"""Workload-level parity: the whole path (score -> head sum -> top-k ->
sparse attention, with the focal-layer schedule) against the oracle on the
seeded synthetic workloads.

Kept sets are accepted when they differ from the oracle's only inside the
1e-6 relative tie band around the k-th oracle score.  Such a set is then a
correct selection, and the layers that reuse it are checked against the
oracle's attention over that same validated set (with the oracle's own set
whenever the two agree, which is the common case).
"""
import math

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


def kvsel():
    from decode_focal_layer_amd import kvsel as m
    return m


def focal_kvs(w, t=0, shared_rows=None):
    """Per-layer views; a shared prefix is declared cacheable unless
    shared_rows says otherwise (the hint does not change results)."""
    kv = kvsel()
    cfg = w.cfg
    max_len = int(w.seq_len_np.max())
    if shared_rows is None:
        shared_rows = cfg.prefix_len if cfg.shared_prefix else 0
    return [kv.KV(w.k_pool[l], w.v_pool[l], w.block_table, w.seq_len[t], w.seg_begin, w.seg_end,
                  max_seq_len=max_len, max_seg_len=cfg.n_visual, min_seg_len=cfg.n_visual,
                  shared_rows=shared_rows)
            for l in range(cfg.layers)]


def test_c0_full():
    """One decode step at the C0 shape: dense attention, focal scores, top-179,
    gathered sparse attention over the kept visual rows plus the 512 text rows."""
    kv = kvsel()
    cfg = synth.C0
    w = gen.make_focal(cfg, DEV)
    k = cfg.k
    assert k == 179
    kvd = focal_kvs(w)[0]
    q = w.q[0, 0].contiguous()
    out = torch.zeros((1, 16, 128), dtype=torch.float32, device=DEV)
    lse = torch.zeros((1, 16), dtype=torch.float32, device=DEV)
    sc = torch.zeros((1, 8, cfg.n_visual), dtype=torch.float32, device=DEV)
    idx = torch.zeros((1, 8, k), dtype=torch.int32, device=DEV)
    out_s = torch.zeros_like(out)
    kv.dense_attn(kvd, q, 16, cfg.scale, out, lse, seg_scores=sc)
    kv.topk(sc, cfg.n_visual, k, idx)
    kv.gather_attn(kvd, q, 16, cfg.scale, idx, k, out_s)
    torch.cuda.synchronize()
    kc, vc, qc = w.k_pool[0].cpu(), w.v_pool[0].cpu(), q.cpu()
    n = cfg.prefix_len
    patch = gen.patch_tokens(int(w.patches[0, 0, 0]), int(w.patches[0, 0, 1]), cfg.grid_cols, *cfg.patch)
    hits = 0
    for g in range(8):
        Kl = O.logical_rows(kc, w.table_np[0], g, n)
        Vl = O.logical_rows(vc, w.table_np[0], g, n)
        qg = O.widen(qc[0, 2 * g:2 * g + 2])
        ref, rl = O.dense_attention(qg, Kl, Vl, cfg.scale)
        assert_attn(out[0, 2 * g:2 * g + 2].cpu().numpy(), ref, f"dense g{g}")
        s = O.focal_scores(qg, Kl, 0, cfg.n_visual, cfg.scale)
        gpu_s = sc[0, g].cpu().numpy()
        assert np.abs(gpu_s - s).max() / s.max() < 2e-6
        gi = idx[0, g].cpu().numpy()
        ok, nd = O.tie_band_check(gi, s, k, BAND)
        assert ok, f"g{g}: kept set differs outside the tie band ({nd})"
        hits += len(np.intersect1d(gi, patch))
        refs, _ = O.attention(qg, Kl, Vl, O.kept_rows(gi, 0, cfg.n_visual, n), cfg.scale)
        assert_attn(out_s[0, 2 * g:2 * g + 2].cpu().numpy(), refs, f"sparse g{g}")
    print("patch tokens among the kept:", hits, "of", 8 * len(patch))


def run_schedule(cfg, w, check_every=1, v_scale=1.0, **dec_kw):
    """Run all steps through FocalDecoder; check every layer of every step
    (the absolute error bound taken relative to v_scale)."""
    from decode_focal_layer_amd.decode import FocalDecoder
    kv = kvsel()
    kvs = focal_kvs(w)
    dec = FocalDecoder(kvs, cfg.hq, cfg.k, cfg.focal, cfg.scale, cfg.n_visual, warm_start=cfg.warm_start,
                       device=DEV, **dec_kw)
    kc = [w.k_pool[l].cpu() for l in range(cfg.layers)]
    vc = [w.v_pool[l].cpu() for l in range(cfg.layers)]
    G = cfg.group
    sets = {}          # (t, focal layer) -> validated kept sets [B][hkv][k]
    worst = 0.0
    for t in range(cfg.steps):
        log_case(cfg.name, "step", t)
        dec.step(t, w.q[t], w.seq_len[t])
        torch.cuda.synchronize()
        outs = dec.out.cpu().numpy()
        qc = w.q[t].cpu()
        plan = O.focal_layer_plan(cfg.layers, cfg.focal, t)
        for f in cfg.focal:
            sets[(t, f)] = dec.selection(f).cpu().numpy()
        if t % check_every:
            continue
        for e in plan:
            l = e[1]
            for b in range(cfg.batch):
                n = int(w.seq_len_np[t, b])
                for g in range(cfg.hkv):
                    Kl = O.logical_rows(kc[l], w.table_np[b], g, n)
                    Vl = O.logical_rows(vc[l], w.table_np[b], g, n)
                    qg = O.widen(qc[l, b, g * G:(g + 1) * G])
                    if e[0] in ("dense", "focal"):
                        ref, _ = O.dense_attention(qg, Kl, Vl, cfg.scale)
                        if e[0] == "focal":
                            s = O.focal_scores(qg, Kl, 0, cfg.n_visual, cfg.scale)
                            ok, nd = O.tie_band_check(sets[(t, l)][b, g], s, cfg.k, BAND)
                            assert ok, f"t{t} l{l} b{b} g{g}: kept set outside the tie band ({nd})"
                    else:
                        _, ts, ls = e[1:]
                        rows = O.kept_rows(sets[(ts, ls)][b, g], 0, cfg.n_visual, n)
                        ref, _ = O.attention(qg, Kl, Vl, rows, cfg.scale)
                    ma, _ = assert_attn(outs[l, b, g * G:(g + 1) * G] / v_scale, ref / v_scale,
                                        f"t{t} l{l} {e[0]} b{b} g{g}")
                    worst = max(worst, ma)
    print(cfg.name, "worst max-abs error", worst)
    return dec, sets


def test_c1_schedule_small():
    cfg = synth.small(synth.C1, batch=3, layers=6, steps=4, focal=(2, 4), grid_rows=12, grid_cols=32, n_always=80)
    w = gen.make_focal(cfg, DEV)
    run_schedule(cfg, w)


def test_c4_branches_small_cascade():
    """The branched decode with sparse layers split into the shared layout
    rows (once per kv head for all branches) and each branch's own rows,
    merged: every layer of every step against the oracle's attention over
    the union."""
    cfg = synth.small(synth.C4, batch=150, layers=4, steps=2, focal=(1, 2), grid_rows=8, grid_cols=32,
                      n_always=48, suffix_range=(3, 40))
    w = gen.make_focal(cfg, DEV)
    run_schedule(cfg, w, check_every=1, shared_tail=(cfg.n_visual, cfg.prefix_len))


def _c4_wide_shared_v(cfg, w, factor):
    """The workload with the V rows of the shared prefix blocks (the same
    blocks in every table) multiplied by factor in every layer."""
    import dataclasses
    blocks = torch.from_numpy(w.table_np[0, :-(-cfg.prefix_len // 16)].astype(np.int64)).to(DEV)
    vp = []
    for v in w.v_pool:
        v = v.clone()
        v[blocks] = (v[blocks].float() * factor).to(torch.bfloat16)
        vp.append(v)
    vmax = max(float(v.float().abs().max()) for v in vp)
    return dataclasses.replace(w, v_pool=vp), vmax


def test_c4_cascade_shared_rows_beyond_fp16():
    """The branched decode's cascade with the shared prefix's V at 2^17 (about
    1.3e5, beyond fp16) in every layer: every layer of every step, and the
    draft verification cascade, against the oracle (errors relative to the
    largest |V|)."""
    from decode_focal_layer_amd.decode import DraftVerifier
    kv = kvsel()
    cfg = synth.small(synth.C4, batch=150, layers=4, steps=2, focal=(1, 2), grid_rows=8, grid_cols=32,
                      n_always=48, suffix_range=(3, 40))
    w, vmax = _c4_wide_shared_v(cfg, gen.make_focal(cfg, DEV), 2.0 ** 17)
    assert vmax >= 1e5
    run_schedule(cfg, w, check_every=1, v_scale=vmax, shared_tail=(cfg.n_visual, cfg.prefix_len))
    # draft verification over layer 0, shared rows folded in
    m, G, T = 4, cfg.group, cfg.steps
    n_np = w.seq_len_np[T - 1].astype(np.int64)
    kvd = kv.KV(w.k_pool[0], w.v_pool[0], w.block_table, w.seq_len[T - 1], w.seg_begin, w.seg_end,
                max_seq_len=int(n_np.max()), max_seg_len=cfg.n_visual, min_seg_len=cfg.n_visual,
                shared_rows=cfg.prefix_len)
    g = torch.Generator(device=DEV).manual_seed(cfg.seed + 91)
    keys = torch.rand((cfg.batch * cfg.hkv, cfg.n_visual), generator=g, device=DEV)
    idx = keys.argsort(dim=1)[:, :cfg.k].sort(dim=1).values.to(torch.int32).view(cfg.batch, cfg.hkv, cfg.k)
    q = torch.randn((cfg.batch, m, cfg.hq, 128), generator=g, device=DEV).to(torch.bfloat16)
    out = torch.empty((cfg.batch, m, cfg.hq, 128), dtype=torch.float32, device=DEV)
    lse = torch.empty((cfg.batch, m, cfg.hq), dtype=torch.float32, device=DEV)
    log_case("c4-verify-wide-v", cfg.batch, m)
    DraftVerifier(kvd, m, cfg.hq, cfg.scale, shared_tail=(cfg.n_visual, cfg.prefix_len),
                  device=DEV).verify(q, idx, cfg.k, out, lse)
    torch.cuda.synchronize()
    idx_c, q_c, vc = idx.cpu().numpy(), q.cpu(), w.v_pool[0].cpu()
    rng = np.random.default_rng(93)
    for _ in range(16):
        b, h = int(rng.integers(cfg.batch)), int(rng.integers(cfg.hkv))
        n = int(n_np[b])
        Kl = O.logical_rows(w.k_pool[0].cpu(), w.table_np[b], h, n)
        Vl = O.logical_rows(vc, w.table_np[b], h, n)
        rows = O.kept_rows(idx_c[b, h], 0, cfg.n_visual, n)
        ref, rl = O.verify_attention(O.widen(q_c[b, :, h * G:(h + 1) * G]), Kl, Vl, rows, n, cfg.scale)
        got = out[b, :, h * G:(h + 1) * G].cpu().numpy()
        assert_attn(got.reshape(-1, 128) / vmax, ref.reshape(-1, 128) / vmax, f"c4 verify wide-v b{b} g{h}")
        assert np.abs(lse[b, :, h * G:(h + 1) * G].cpu().numpy() - rl).max() < 1e-4


def test_c4_branches_small_and_shared_prefix_equals_private_copy():
    cfg = synth.small(synth.C4, batch=6, layers=5, steps=3, focal=(1, 3), grid_rows=8, grid_cols=32,
                      n_always=32, suffix_range=(3, 40))
    w = gen.make_focal(cfg, DEV)
    dec, sets = run_schedule(cfg, w)
    out_shared = dec.out.clone()
    # private copy of the prefix for every branch: same rows, different blocks
    pref = cfg.prefix_len // 16
    B = cfg.batch
    tab = w.table_np.copy()
    extra = []
    for b in range(B):
        new = w.num_blocks + b * pref + np.arange(pref)
        tab[b, :pref] = new
        extra.append(new)
    kp = [torch.cat([w.k_pool[l]] + [w.k_pool[l][:pref]] * B) for l in range(cfg.layers)]
    vp = [torch.cat([w.v_pool[l]] + [w.v_pool[l][:pref]] * B) for l in range(cfg.layers)]
    w2 = gen.FocalWorkload(cfg=cfg, k_pool=kp, v_pool=vp, block_table=torch.from_numpy(tab).to(DEV), q=w.q,
                           seq_len=w.seq_len, seg_begin=w.seg_begin, seg_end=w.seg_end, table_np=tab,
                           seq_len_np=w.seq_len_np, patches=w.patches, suffix_len=w.suffix_len,
                           num_blocks=w.num_blocks + B * pref, max_blocks=w.max_blocks)
    from decode_focal_layer_amd.decode import FocalDecoder
    # the private copy streams every row (no shared-prefix hint)
    dec2 = FocalDecoder(focal_kvs(w2, shared_rows=0), cfg.hq, cfg.k, cfg.focal, cfg.scale, cfg.n_visual, device=DEV)
    for t in range(cfg.steps):
        dec2.step(t, w.q[t], w.seq_len[t])
    torch.cuda.synchronize()
    assert (dec2.out - out_shared).abs().max().item() < 1e-5   # summation order only
    for f in cfg.focal:
        assert torch.equal(dec2.selection(f), dec.selection(f))



@pytest.mark.parametrize("cascade", [False, True])
def test_deterministic_flag_bitwise_at_full_shape(cascade):
    """KVSEL_FLAG_DETERMINISTIC: two runs of 3 decode steps at a full shape
    -- the FastOCR decode (28 layers, batch 32, 7424-row caches) or the
    branched decode's cascade (512 branches over the shared prefix) -- give
    bitwise equal outputs and kept sets, and the same outputs as the default
    mode within the rounding of the row order."""
    from decode_focal_layer_amd import kvsel
    from decode_focal_layer_amd.decode import FocalDecoder
    cfg = synth.small(synth.C4 if cascade else synth.C1, steps=3)
    w = gen.make_focal(cfg, DEV)
    max_len = int(w.seq_len_np.max())
    runs = {}
    for det, rep in ((True, 0), (True, 1), (False, 0)):
        kvs = [kvsel.KV(w.k_pool[l], w.v_pool[l], w.block_table, w.seq_len[0], w.seg_begin, w.seg_end,
                        max_seq_len=max_len, max_seg_len=cfg.n_visual, min_seg_len=cfg.n_visual,
                        shared_rows=cfg.prefix_len if cascade else 0, deterministic=det)
               for l in range(cfg.layers)]
        dec = FocalDecoder(kvs, cfg.hq, cfg.k, cfg.focal, cfg.scale, cfg.n_visual, device=DEV,
                           shared_tail=(cfg.n_visual, cfg.prefix_len) if cascade else None)
        outs, sets = [], []
        log_case("deterministic", cascade, det, rep)
        for t in range(cfg.steps):
            dec.step(t, w.q[t], w.seq_len[t])
            outs.append(dec.out.clone())
            sets.append(torch.stack([dec.selection(f).clone() for f in cfg.focal]))
        torch.cuda.synchronize()
        runs[(det, rep)] = (torch.stack(outs).cpu(), torch.stack(sets).cpu())
    (o1, s1), (o2, s2), (o3, s3) = runs[(True, 0)], runs[(True, 1)], runs[(False, 0)]
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    assert torch.equal(s1, s3)
    assert (o1 - o3).abs().max().item() < 1e-5
