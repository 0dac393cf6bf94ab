"""Full-size parity of the FastKV propagation layer (C2, in full), of the
focal-layer profiling run on the FastOCR cache, and of draft verification at
the branched-decode size, in the launch configuration the benchmark times.
The multi-step decodes have modules of their own (test_gpu_full_c1/c3/c4)."""
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
