"""Per-entry-point parity of libkvsel against the oracle on small seeded
shapes that span several tiles and ragged tails, with edge cases."""
import ctypes
import math

import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests.gpu_util import (assert_attn, attn_errors, cpu_pool, log_case, need_gpu, random_paged, rel_err, BAND)

pytestmark = pytest.mark.gpu
DEV = "cuda"
SCALE = 1.0 / math.sqrt(128)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def K():
    from decode_focal_layer_amd import kvsel
    return kvsel


def make_kv(rng, batch, hkv, lens, segs, max_len=None):
    kvsel = K()
    max_len = max_len or max(lens)
    kp, vp, table = random_paged(rng, batch, hkv, max_len, DEV)
    seg_b = np.array([s[0] for s in segs], dtype=np.int32)
    seg_e = np.array([s[1] for s in segs], dtype=np.int32)
    kv = kvsel.KV(kp, vp, torch.from_numpy(table).to(DEV), torch.tensor(lens, dtype=torch.int32, device=DEV),
                  torch.from_numpy(seg_b).to(DEV), torch.from_numpy(seg_e).to(DEV),
                  max_seq_len=max_len, max_seg_len=int((seg_e - seg_b).max()), min_seg_len=int((seg_e - seg_b).min()))
    return kv, cpu_pool(kp), cpu_pool(vp), table


ATTN_CASES = [(1, 1, [1]), (2, 2, [15, 16]), (4, 1, [17]), (8, 2, [300, 33]), (2, 3, [4095, 1000, 2]),
              (2, 1, [8193]), (4, 2, [1, 1000]),
              (3, 2, [300, 33]), (5, 1, [1000]), (6, 2, [17, 4095]), (7, 1, [129])]


@pytest.mark.parametrize("G,batch,lens", ATTN_CASES)
def test_dense_and_gather_attention(G, batch, lens):
    kvsel = K()
    rng = np.random.default_rng(G * 100 + len(lens))
    hkv = 2
    hq = hkv * G
    segs = [(min(3, n), max(min(3, n), n - min(5, n // 3))) for n in lens]
    kv, kc, vc, table = make_kv(rng, batch, hkv, lens, segs)
    q = torch.randn((batch, hq, 128), generator=torch.Generator().manual_seed(7)).to(torch.bfloat16).to(DEV)
    out = torch.zeros((batch, hq, 128), dtype=torch.float32, device=DEV)
    lse = torch.zeros((batch, hq), dtype=torch.float32, device=DEV)
    log_case("dense", G, lens)
    kvsel.dense_attn(kv, q, hq, SCALE, out, lse)
    seg_lens = [s1 - s0 for s0, s1 in segs]
    kmax = max(1, min(seg_lens))
    idx_np = np.zeros((batch, hkv, kmax), dtype=np.int32)
    for b in range(batch):
        for g in range(hkv):
            sl = seg_lens[b]
            pick = np.sort(rng.choice(sl, size=min(kmax, sl), replace=False)) if sl else np.array([], np.int64)
            row = np.full(kmax, -1, dtype=np.int32)       # -1: skipped (outside the segment)
            row[: len(pick)] = pick
            idx_np[b, g] = row
    idx = torch.from_numpy(idx_np).to(DEV)
    out_s = torch.zeros_like(out)
    lse_s = torch.zeros_like(lse)
    log_case("gather", G, lens, kmax)
    kvsel.gather_attn(kv, q, hq, SCALE, idx, kmax, out_s, lse_s)
    torch.cuda.synchronize()
    qc = q.cpu()
    for b in range(batch):
        for g in range(hkv):
            Kl = O.logical_rows(kc, table[b], g, lens[b])
            Vl = O.logical_rows(vc, table[b], g, lens[b])
            qg = O.widen(qc[b, g * G:(g + 1) * G])
            ref, rl = O.dense_attention(qg, Kl, Vl, SCALE)
            assert_attn(out[b, g * G:(g + 1) * G].cpu().numpy(), ref, f"dense b{b} g{g}")
            assert np.abs(lse[b, g * G:(g + 1) * G].cpu().numpy() - rl).max() < 1e-4
            sel = idx_np[b, g][idx_np[b, g] >= 0]
            rows = O.kept_rows(sel, segs[b][0], segs[b][1], lens[b])
            ref_s, rl_s = O.attention(qg, Kl, Vl, rows, SCALE)
            assert_attn(out_s[b, g * G:(g + 1) * G].cpu().numpy(), ref_s, f"gather b{b} g{g}")
            assert np.abs(lse_s[b, g * G:(g + 1) * G].cpu().numpy() - rl_s).max() < 1e-4


# (G, batch, lens, segments): split (few pairs) and one work-group per pair,
# ragged lengths, empty and whole segments
MASS_CASES = [(1, 1, [1], [(0, 1)]), (2, 2, [17, 300], [(3, 15), (0, 300)]),
              (4, 3, [4095, 1000, 2], [(100, 4000), (7, 7), (1, 2)]), (8, 1, [8193], [(0, 8000)]),
              (2, 32, None, None), (3, 2, [17, 300], [(3, 15), (0, 300)]), (6, 1, [1000], [(5, 900)])]


@pytest.mark.parametrize("G,batch,lens,segs", MASS_CASES)
def test_visual_mass(G, batch, lens, segs):
    """The image-attention ratio per head against the oracle (fp32 sums:
    absolute error <= 1e-5 on a value in [0, 1]); V is not needed."""
    kvsel = K()
    rng = np.random.default_rng(700 + G * batch)
    hkv = 8 if batch == 32 else 2
    if lens is None:
        lens = [int(x) for x in rng.integers(200, 900, size=batch)]
        segs = [(int(rng.integers(0, 50)), n - int(rng.integers(0, 100))) for n in lens]
    hq = hkv * G
    kv, kc, _, table = make_kv(rng, batch, hkv, lens, segs)
    kv = kvsel.KV(kv.k_pool, None, kv.block_table, kv.seq_len, kv.seg_begin, kv.seg_end,
                  max_seq_len=kv.max_seq_len, max_seg_len=kv.max_seg_len, min_seg_len=kv.min_seg_len)
    q = (torch.randn((batch, hq, 128), generator=torch.Generator().manual_seed(3)) * 2).to(torch.bfloat16).to(DEV)
    mass = torch.full((batch, hq), -1.0, dtype=torch.float32, device=DEV)
    log_case("visual_mass", G, batch, lens[:4])
    kvsel.visual_mass(kv, q, hq, SCALE, mass)
    torch.cuda.synchronize()
    got = mass.cpu().numpy()
    qc = q.cpu()
    for b in range(batch):
        for g in range(hkv):
            Kl = O.logical_rows(kc, table[b], g, lens[b])
            ref = O.visual_mass(O.widen(qc[b, g * G:(g + 1) * G]), Kl, segs[b][0], segs[b][1], SCALE)
            assert np.abs(got[b, g * G:(g + 1) * G] - ref).max() <= 1e-5, f"b{b} g{g}"
    # the whole segment is the whole attention
    assert all(abs(got[b] - 1.0).max() <= 1e-6 for b in range(batch) if segs[b] == (0, lens[b]))


@pytest.mark.parametrize("L,n,quant", [(1, 1, 4), (5, 7, 4), (28, 2048, 64), (100, 33, 0), (1024, 3, 2)])
def test_pick_layers(L, n, quant):
    """Exact against the oracle on the same fp32 ratios (quantised ratios
    make many equal means: ties go to the lower layer)."""
    kvsel = K()
    rng = np.random.default_rng(L * 7 + n)
    r = rng.random((L, n)).astype(np.float32)
    if quant:
        r = (np.floor(r * quant) / quant).astype(np.float32)
    rt = torch.from_numpy(r).to(DEV)
    for n_pick in sorted({1, min(2, L), max(1, L // 3), L}):
        out = torch.full((n_pick,), -1, dtype=torch.int32, device=DEV)
        kvsel.pick_layers(rt, n_pick, out)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), O.pick_focal_layers(r.astype(np.float64), n_pick)), n_pick


def test_pick_layers_exact_sums():
    """Ranking by exact sums, independent of the order of the terms: layers
    holding the same ratios in different orders tie (lower layer first); a
    layer whose sum is larger by 2^-60 -- far below the rounding of any fp64
    sum of 2048 ratios -- ranks first, one smaller by 2^-60 last."""
    kvsel = K()
    rng = np.random.default_rng(77)
    base = rng.random(2048).astype(np.float32)
    ratios = np.stack([base, rng.permutation(base), base[::-1], base, rng.permutation(base), base])
    ratios = np.concatenate([ratios, np.zeros((6, 1), np.float32)], axis=1).astype(np.float32)
    tiny = np.float32(2.0 ** -60)
    ratios[3, -1] = tiny                   # exact sum: base's + 2^-60
    ratios[5, -1] = -tiny                  # exact sum: base's - 2^-60
    r64 = ratios.astype(np.float64)
    assert list(O.pick_focal_layers(r64, 1)) == [3]
    assert list(O.pick_focal_layers(r64, 5)) == [0, 1, 2, 3, 4]
    rt = torch.from_numpy(np.ascontiguousarray(ratios)).to(DEV)
    for n_pick in range(1, 7):
        out = torch.full((n_pick,), -1, dtype=torch.int32, device=DEV)
        kvsel.pick_layers(rt, n_pick, out)
        torch.cuda.synchronize()
        want = O.pick_focal_layers(r64, n_pick)
        assert np.array_equal(out.cpu().numpy(), want), (n_pick, out.cpu().numpy(), want)


@pytest.mark.parametrize("G", [2, 4])
def test_split_merge_repeated_launches(G):
    """Pairs whose rows are split over many work-groups (18 here) are merged
    by the last of their work-groups to finish.  Launches back to back on one
    stream with the deterministic row order sum the same terms in the same
    order, so every launch's output is bitwise equal to the first -- a merge
    that read a record before it was complete, or a counter left non-zero by
    an earlier launch, would break that -- and matches the oracle; the
    workspace's arrival counters are zero afterwards."""
    kvsel = K()
    rng = np.random.default_rng(900 + G)
    hkv, batch = 2, 2
    hq = hkv * G
    lens = [6000, 3333]
    segs = [(100, 5900), (0, 3000)]
    kv0, kc, vc, table = make_kv(rng, batch, hkv, lens, segs)
    kv = kvsel.KV(kv0.k_pool, kv0.v_pool, kv0.block_table, kv0.seq_len, kv0.seg_begin, kv0.seg_end,
                  kv0.max_seq_len, kv0.max_seg_len, kv0.min_seg_len, 0, True)
    q = torch.randn((batch, hq, 128), generator=torch.Generator().manual_seed(31)).to(torch.bfloat16).to(DEV)
    k = 1500
    idx_np = np.stack([np.stack([np.sort(rng.choice(s1 - s0, size=k, replace=False)) for _ in range(hkv)])
                       for s0, s1 in segs]).astype(np.int32)
    idx = torch.from_numpy(idx_np).to(DEV)
    ws = kvsel.Workspace(DEV)
    log_case("split-merge", G)
    gathered = [torch.zeros((batch, hq, 128), dtype=torch.float32, device=DEV) for _ in range(16)]
    dense = [torch.zeros((batch, hq, 128), dtype=torch.float32, device=DEV) for _ in range(8)]
    for i, o in enumerate(gathered):
        kvsel.gather_attn(kv, q, hq, SCALE, idx, k, o, ws=ws)
        if i % 2 == 0:
            kvsel.dense_attn(kv, q, hq, SCALE, dense[i // 2], ws=ws)
    torch.cuda.synchronize()
    for o in gathered[1:]:
        assert torch.equal(o, gathered[0])
    for o in dense[1:]:
        assert torch.equal(o, dense[0])
    qc = q.cpu()
    for b in range(batch):
        for g in range(hkv):
            Kl = O.logical_rows(kc, table[b], g, lens[b])
            Vl = O.logical_rows(vc, table[b], g, lens[b])
            qg = O.widen(qc[b, g * G:(g + 1) * G])
            ref_d, _ = O.dense_attention(qg, Kl, Vl, SCALE)
            assert_attn(dense[0][b, g * G:(g + 1) * G].cpu().numpy(), ref_d, f"dense b{b} g{g}")
            rows = O.kept_rows(idx_np[b, g], segs[b][0], segs[b][1], lens[b])
            ref_s, _ = O.attention(qg, Kl, Vl, rows, SCALE)
            assert_attn(gathered[0][b, g * G:(g + 1) * G].cpu().numpy(), ref_s, f"gather b{b} g{g}")
    addr = ws.buf.data_ptr()
    pad = (-addr) % 256
    assert int(ws.buf[pad:pad + 65536].count_nonzero().item()) == 0


def test_gather_full_budget_equals_dense_and_empty_rows():
    kvsel = K()
    rng = np.random.default_rng(11)
    lens = [700, 64]
    segs = [(0, 700), (0, 64)]
    kv, kc, vc, table = make_kv(rng, 2, 2, lens, segs)
    hq = 4
    q = torch.randn((2, hq, 128), generator=torch.Generator().manual_seed(3)).to(torch.bfloat16).to(DEV)
    d = torch.zeros((2, hq, 128), dtype=torch.float32, device=DEV)
    kvsel.dense_attn(kv, q, hq, SCALE, d)
    # k = segment length: every row kept
    idx = torch.full((2, 2, 700), -1, dtype=torch.int32)
    idx[0] = torch.arange(700, dtype=torch.int32)
    idx[1, :, :64] = torch.arange(64, dtype=torch.int32)
    s = torch.zeros_like(d)
    kvsel.gather_attn(kv, q, hq, SCALE, idx.to(DEV), 700, s)
    torch.cuda.synchronize()
    assert attn_errors(s.cpu().numpy(), d.cpu().numpy())[0] < 1e-5
    # k = 0 and nothing outside the segment: no rows -> out = 0, lse = -inf
    z = torch.ones_like(d)
    lse = torch.zeros((2, hq), dtype=torch.float32, device=DEV)
    kvsel.gather_attn(kv, q, hq, SCALE, None, 0, z, lse)
    torch.cuda.synchronize()
    assert torch.all(z == 0) and torch.all(torch.isinf(lse) & (lse < 0))


@pytest.mark.parametrize("n,k", [(3072, 154), (40000, 2048)])
def test_topk_rows_of_their_own_length(n, k):
    """n_per_row: each row ranks its own first n_r scores (clamped to [0, n]);
    a row with at most k candidates gets them all, then -1.  Rows: full,
    shorter, exactly k, fewer than k, zero, negative, above n; warm-started
    rows (warm indices inside the row) give the same."""
    kvsel = K()
    rng = np.random.default_rng(n + 17)
    counts = np.array([n, n - 37, k, k - 3, 0, -5, n + 100, n // 2], dtype=np.int32)
    rows = len(counts)
    s = (rng.integers(0, 400, size=(rows, n)) / 400).astype(np.float32)   # ties included
    st = torch.from_numpy(s).to(DEV)
    nr = torch.from_numpy(counts).to(DEV)
    idx = torch.full((rows, k), -7, dtype=torch.int32, device=DEV)
    log_case("topk-rows", n, k)
    kvsel.topk(st, n, k, idx, n_per_row=nr)
    warm = np.zeros((rows, k), dtype=np.int32)
    for r in range(rows):
        nr_ = min(max(int(counts[r]), 0), n)
        warm[r] = np.sort(rng.choice(nr_, size=k, replace=False)) if nr_ > k else np.arange(k)
    idx_w = torch.full((rows, k), -7, dtype=torch.int32, device=DEV)
    kvsel.topk(st, n, k, idx_w, warm=torch.from_numpy(warm).to(DEV), n_per_row=nr)
    torch.cuda.synchronize()
    got, got_w = idx.cpu().numpy(), idx_w.cpu().numpy()
    for r in range(rows):
        nr_ = min(max(int(counts[r]), 0), n)
        if nr_ > k:
            want = O.topk(s[r, :nr_], k)
        else:
            want = np.concatenate([np.arange(nr_), np.full(k - nr_, -1)])
        assert np.array_equal(got[r], want), f"row {r} (n_r {counts[r]})"
        assert np.array_equal(got_w[r], want), f"warm row {r} (n_r {counts[r]})"


@pytest.mark.parametrize("n,k,mode", [(1, 1, "rand"), (5, 3, "ties"), (64, 64, "rand"), (3584, 179, "rand"),
                                      (6400, 320, "ties"), (3072, 154, "equal"), (12288, 600, "rand"),
                                      (12289, 7, "ties"), (32760, 6554, "rand"), (40000, 2048, "ties"),
                                      # every score equal, a narrow band of scores, k = 1, k = n - 1,
                                      # k = n, a row read from global memory on every pass
                                      (40000, 5000, "equal"), (30000, 3000, "narrow"), (20000, 1, "rand"),
                                      (20000, 19999, "ties"), (20000, 20000, "rand"), (131072, 2048, "rand"),
                                      # scores over many exponents, both signs, and a k-th score in the
                                      # highest occupied coarse bin
                                      (50000, 1000, "wide"), (50000, 300, "signed"), (16384, 3, "spike"),
                                      # the coarse bin of the k-th score taken whole
                                      (16384, 5, "spike"),
                                      # the edges of the register-held row sizes (4, 8, 16, 32 keys per
                                      # thread) and the first row past them
                                      (4096, 100, "wide"), (4097, 4000, "ties"), (32768, 4000, "signed"),
                                      (32769, 100, "wide"),
                                      # the longest row staged in LDS and the first read from global memory
                                      (36864, 1000, "wide"), (36865, 1000, "ties")])
def test_topk_exact(n, k, mode):
    kvsel = K()
    rng = np.random.default_rng(n + k)
    rows = 3
    if mode == "rand":
        s = rng.random((rows, n)).astype(np.float32) * 1e-3
    elif mode == "ties":
        s = (rng.integers(0, 50, size=(rows, n)) / 50).astype(np.float32)
    elif mode == "narrow":
        s = (1.0 + rng.random((rows, n)) * 1e-3).astype(np.float32)
    elif mode == "wide":
        s = np.exp(rng.standard_normal((rows, n)) * 8.0).astype(np.float32)
    elif mode == "signed":
        s = rng.standard_normal((rows, n)).astype(np.float32)
    elif mode == "spike":
        s = (rng.random((rows, n)) * 1e-6).astype(np.float32)
        s[:, rng.choice(n, size=5, replace=False)] = np.float32(0.5)
    else:
        s = np.full((rows, n), 1.0 / n, dtype=np.float32)
    ld = n + 5
    sp = np.zeros((rows, ld), dtype=np.float32)
    sp[:, :n] = s
    sp[:, n:] = 99.0       # past n: never selected
    st = torch.from_numpy(sp).to(DEV)
    idx = torch.full((rows, k), -7, dtype=torch.int32, device=DEV)
    log_case("topk", n, k, mode)
    kvsel.topk(st, n, k, idx)
    # warm start from a random valid set, and from an invalid one (ranked cold)
    warm = np.stack([np.sort(rng.choice(n, size=k, replace=False)) for _ in range(rows)]).astype(np.int32)
    if k > 1:
        warm[1, 0], warm[1, 1] = warm[1, 1], warm[1, 0]      # not ascending
    idx_w = torch.full((rows, k), -7, dtype=torch.int32, device=DEV)
    kvsel.topk(st, n, k, idx_w, warm=torch.from_numpy(warm).to(DEV))
    torch.cuda.synchronize()
    got, got_w = idx.cpu().numpy(), idx_w.cpu().numpy()
    for r in range(rows):
        want = O.topk(s[r], k)
        assert np.array_equal(got[r], want), f"row {r}"
        assert np.array_equal(got_w[r], want), f"warm row {r}"


# pool widths: none, FastKV's 7, the widest staged through LDS (511) and one past it
@pytest.mark.parametrize("norm,reduce,pool", [(0, 0, 1), (1, 0, 1), (0, 1, 1), (1, 0, 7), (0, 1, 7), (0, 0, 511),
                                              (1, 1, 513)])
def test_decode_scores(norm, reduce, pool):
    kvsel = K()
    rng = np.random.default_rng(norm * 10 + reduce * 3 + pool)
    lens = [900, 1500]
    segs = [(50, 850), (0, 1400)]
    kv, kc, vc, table = make_kv(rng, 2, 4, lens, segs)
    G, hq = 2, 8
    q = torch.randn((2, 1, hq, 128), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).to(DEV)
    nout = 4 if reduce == 0 else 1
    ld = 1410
    sc = torch.full((2, nout, ld), -1.0, dtype=torch.float32, device=DEV)
    log_case("score", norm, reduce, pool)
    kvsel.score(kv, q, 1, hq, SCALE, reduce, norm, True, pool, sc)
    torch.cuda.synchronize()
    got = sc.cpu().numpy()
    qc = q.cpu()
    nm = "segment" if norm == 0 else "context"
    worst = 0.0
    for b in range(2):
        s0, s1 = segs[b]
        parts = []
        for g in range(4):
            Kl = O.logical_rows(kc, table[b], g, lens[b])
            parts.append(O.focal_scores(O.widen(qc[b, 0, g * G:(g + 1) * G]), Kl, s0, s1, SCALE, nm))
        refs = parts if reduce == 0 else [np.sum(parts, axis=0)]
        for o, ref in enumerate(refs):
            if pool > 1:
                ref = O.avg_pool(ref, pool)
            worst = max(worst, rel_err(got[b, o, : s1 - s0], ref))
            assert np.all(got[b, o, s1 - s0:] == -1.0)
    print("max relative score error", worst)
    assert worst < 2e-6


# Long segments, eight pooled rows: the pool then takes several positions per
# thread (65536 positions: two; 262144: eight), at the widest halo it stages
# through LDS.  Same scores as the oracle's pool over its focal scores.
@pytest.mark.parametrize("n,pool", [(65536, 511), (262144, 511), (262144, 7)])
def test_decode_scores_long_pooled(n, pool):
    kvsel = K()
    rng = np.random.default_rng(n + pool)
    hkv, G = 8, 2
    hq = hkv * G
    kv, kc, vc, table = make_kv(rng, 1, hkv, [n], [(0, n)])
    q = torch.randn((1, 1, hq, 128), generator=torch.Generator().manual_seed(11)).to(torch.bfloat16).to(DEV)
    sc = torch.full((1, hkv, n), -1.0, dtype=torch.float32, device=DEV)
    log_case("score long pooled", n, pool)
    kvsel.score(kv, q, 1, hq, SCALE, 0, 0, True, pool, sc)
    torch.cuda.synchronize()
    got = sc.cpu().numpy()
    qc = q.cpu()
    worst = 0.0
    for g in range(hkv):
        Kl = O.logical_rows(kc, table[0], g, n)
        ref = O.avg_pool(O.focal_scores(O.widen(qc[0, 0, g * G:(g + 1) * G]), Kl, 0, n, SCALE, "segment"), pool)
        worst = max(worst, rel_err(got[0, g], ref))
    print("max relative score error", worst)
    assert worst < 2e-6


def test_dense_fused_scores_match_score_call():
    kvsel = K()
    rng = np.random.default_rng(21)
    lens = [4096, 3000]
    segs = [(0, 3584), (0, 2500)]
    kv, kc, vc, table = make_kv(rng, 2, 8, lens, segs)
    hq = 16
    q = torch.randn((2, hq, 128), generator=torch.Generator().manual_seed(9)).to(torch.bfloat16).to(DEV)
    out = torch.zeros((2, hq, 128), dtype=torch.float32, device=DEV)
    s1 = torch.zeros((2, 8, 3584), dtype=torch.float32, device=DEV)
    s2 = torch.zeros_like(s1)
    kvsel.dense_attn(kv, q, hq, SCALE, out, seg_scores=s1)
    kvsel.score(kv, q.view(2, 1, hq, 128), 1, hq, SCALE, 0, 0, True, 1, s2)
    torch.cuda.synchronize()
    assert torch.equal(s1[0], s2[0]) and torch.equal(s1[1, :, :2500], s2[1, :, :2500])


# (G, norm, batch, hkv, len, seg): few pairs -> split attention + separate select;
# >= 256 (G <= 2) or 512 (G = 4) pairs -> the one-kernel fused focal pass
FOCAL_CASES = [(2, 0, 3, 4, 3000, 2500), (4, 1, 3, 4, 3000, 2500), (1, 0, 3, 4, 3000, 2500), (8, 0, 3, 4, 3000, 2500),
               (2, 0, 32, 8, 900, 700), (4, 0, 64, 8, 520, 400), (1, 0, 32, 8, 400, 333),
               (3, 0, 3, 4, 3000, 2500), (5, 1, 3, 4, 3000, 2500), (6, 0, 8, 4, 900, 700), (7, 0, 3, 4, 400, 333),
               # one work-group per pair (the fused kernel): a segment whose G x 10240 logits fill the fused
               # kernel's 80 KiB of LDS exactly, and one row more (attention with logits, then the selection)
               (2, 0, 32, 8, 10300, 10240), (2, 0, 32, 8, 10300, 10241)]


@pytest.mark.parametrize("G,norm,batch,hkv,n,seg", FOCAL_CASES)
def test_focal_attn_equals_dense_then_topk(G, norm, batch, hkv, n, seg):
    """The focal pass gives the same scores and kept set as dense attention
    with scores followed by the standalone top-k (bit for bit), and the same
    out and lse up to summation order."""
    kvsel = K()
    rng = np.random.default_rng(31 + G + batch)
    hq = hkv * G
    lens = [n - (b % 3) * 7 for b in range(batch)]
    segs = [(0, seg)] * batch
    kv, kc, vc, table = make_kv(rng, batch, hkv, lens, segs)
    q = torch.randn((batch, hq, 128), generator=torch.Generator().manual_seed(4)).to(torch.bfloat16).to(DEV)
    k = max(1, seg // 20)
    o1, o2 = (torch.zeros((batch, hq, 128), dtype=torch.float32, device=DEV) for _ in range(2))
    l1, l2 = (torch.zeros((batch, hq), dtype=torch.float32, device=DEV) for _ in range(2))
    s1, s2 = (torch.zeros((batch, hkv, seg), dtype=torch.float32, device=DEV) for _ in range(2))
    i1, i2, i3, i4 = (torch.zeros((batch, hkv, k), dtype=torch.int32, device=DEV) for _ in range(4))
    log_case("focal", G, norm, batch, hkv, n, seg)
    kvsel.dense_attn(kv, q, hq, SCALE, o1, l1, seg_scores=s1, norm=norm)
    kvsel.topk(s1, seg, k, i1)
    kvsel.focal_attn(kv, q, hq, SCALE, o2, k, i2, lse=l2, seg_scores=s2, norm=norm)
    kvsel.focal_attn(kv, q, hq, SCALE, o2, k, i3, warm=i1, norm=norm)     # warm start: same set
    kvsel.focal_attn(kv, q, hq, SCALE, o2, k, i4, norm=norm)              # without the score output
    torch.cuda.synchronize()
    # scores and kept sets bit for bit; out and lse up to the rounding of the
    # order in which the waves took their rows
    assert torch.equal(s1, s2)
    assert torch.equal(i1, i2) and torch.equal(i1, i3) and torch.equal(i1, i4)
    assert (o1 - o2).abs().max().item() < 1e-5 and (l1 - l2).abs().max().item() < 1e-5
    qc = q.cpu()
    nm = "segment" if norm == 0 else "context"
    for b in range(0, batch, max(1, batch // 3)):
        for g in range(hkv):
            Kl = O.logical_rows(kc, table[b], g, lens[b])
            Vl = O.logical_rows(vc, table[b], g, lens[b])
            qg = O.widen(qc[b, g * G:(g + 1) * G])
            ref = O.focal_scores(qg, Kl, 0, seg, SCALE, nm)
            ok, nd = O.tie_band_check(i2[b, g].cpu().numpy(), ref, k, BAND)
            assert ok, (b, g, nd)
            assert rel_err(s2[b, g].cpu().numpy(), ref) < 2e-6
            refo, _ = O.dense_attention(qg, Kl, Vl, SCALE)
            assert_attn(o2[b, g * G:(g + 1) * G].cpu().numpy(), refo, f"focal out b{b} g{g}")


@pytest.mark.parametrize("G,W,reduce,causal", [(4, 8, 1, True), (4, 8, 0, True), (2, 8, 0, False), (1, 5, 1, True),
                                              (3, 8, 0, True), (5, 6, 1, False), (6, 5, 0, True), (7, 4, 1, True),
                                              # more than 32 query rows per kv head: blocks of 32 (2, 3 and 16)
                                              (8, 8, 1, True), (8, 8, 0, False), (5, 13, 1, True), (8, 64, 0, True)])
def test_window_scores(G, W, reduce, causal):
    kvsel = K()
    rng = np.random.default_rng(G * 7 + W)
    hkv = 3
    hq = hkv * G
    lens = [2085, 1200]
    segs = [(0, 2085 - W), (0, 1200 - W)]
    kv, kc, vc, table = make_kv(rng, 2, hkv, lens, segs)
    q = torch.randn((2, W, hq, 128), generator=torch.Generator().manual_seed(13)).to(torch.bfloat16).to(DEV)
    nout = hkv if reduce == 0 else 1
    ld = 2100
    sc = torch.full((2, nout, ld), -1.0, dtype=torch.float32, device=DEV)
    log_case("window", G, W, reduce, causal)
    kvsel.score(kv, q, W, hq, SCALE, reduce, 1, causal, 7, sc)
    torch.cuda.synchronize()
    got = sc.cpu().numpy()
    qc = q.cpu()
    worst = 0.0
    for b in range(2):
        s0, s1 = segs[b]
        parts = []
        for g in range(hkv):
            Kl = O.logical_rows(kc, table[b], g, lens[b])
            qw = O.widen(qc[b, :, g * G:(g + 1) * G])
            parts.append(O.window_scores(qw, Kl, s0, s1, SCALE, causal))
        refs = parts if reduce == 0 else [np.sum(parts, axis=0)]
        for o, ref in enumerate(refs):
            ref = O.avg_pool(ref, 7)
            worst = max(worst, rel_err(got[b, o, : s1 - s0], ref))
            assert np.all(got[b, o, s1 - s0:] == -1.0)
            k = max(1, (s1 - s0) // 5)
            idx = torch.zeros((1, k), dtype=torch.int32, device=DEV)
            kvsel.topk(sc[b, o:o + 1, :].contiguous(), s1 - s0, k, idx)
            ok, nd = O.tie_band_check(idx[0].cpu().numpy(), ref, k, BAND)
            assert ok, f"kept set outside tie band ({nd} differ)"
    print("max relative window-score error", worst)
    assert worst < 2e-6


# Window scores of segments starting at rows that are not block aligned, with
# one block of each segment missing from the table (-1): the missing rows take
# no part in any softmax and score 0.  Reference: the oracle's window scores
# over the rows with that block taken out (the window queries and every later
# key move back by 16 together, so what each query sees is unchanged), zeros
# put back in its place, then the pool.
@pytest.mark.parametrize("pool", [1, 7])
def test_window_scores_holed_unaligned(pool):
    import dataclasses
    kvsel = K()
    rng = np.random.default_rng(5150 + pool)
    G, W, hkv = 2, 8, 3
    hq = hkv * G
    lens = [2085, 1200]
    segs = [(37, 2085 - W), (5, 1200 - W)]
    holes = [20, 3]                              # rows 320 .. 335 and 48 .. 63, inside the segments
    kv, kc, vc, table = make_kv(rng, 2, hkv, lens, segs)
    holed = table.copy()
    for b, hb in enumerate(holes):
        holed[b, hb] = -1
    kvh = dataclasses.replace(kv, block_table=torch.from_numpy(holed).to(DEV))
    q = torch.randn((2, W, hq, 128), generator=torch.Generator().manual_seed(17)).to(torch.bfloat16).to(DEV)
    ld = 2100
    sc = torch.full((2, hkv, ld), -1.0, dtype=torch.float32, device=DEV)
    log_case("window holed", pool)
    kvsel.score(kvh, q, W, hq, SCALE, 0, 1, True, pool, sc)
    torch.cuda.synchronize()
    got = sc.cpu().numpy()
    qc = q.cpu()
    worst = 0.0
    for b in range(2):
        s0, s1 = segs[b]
        h0 = 16 * holes[b]
        for g in range(hkv):
            Kl = O.logical_rows(kc, table[b], g, lens[b])
            Kd = np.delete(O.widen(Kl), np.arange(h0, h0 + 16), axis=0)
            qw = O.widen(qc[b, :, g * G:(g + 1) * G])
            part = O.window_scores(qw, Kd, s0, s1 - 16, SCALE, True)
            full = np.concatenate([part[:h0 - s0], np.zeros(16), part[h0 - s0:]])
            ref = O.avg_pool(full, pool) if pool > 1 else full
            if pool == 1:
                assert np.all(got[b, g, h0 - s0:h0 - s0 + 16] == 0.0), (b, g)
            worst = max(worst, rel_err(got[b, g, : s1 - s0], ref))
            assert np.all(got[b, g, s1 - s0:] == -1.0)
    print("max relative window-score error", worst)
    assert worst < 2e-6


def test_gather_rows_exact():
    kvsel = K()
    src = torch.randint(-(1 << 15), 1 << 15, (300, 4096), dtype=torch.int16).view(torch.bfloat16).to(DEV)
    idx = torch.tensor([5, 0, 299, 17, 17, 400, -1], dtype=torch.int32, device=DEV)
    dst = torch.full((7 + 8, 4096), 3.0, dtype=torch.bfloat16, device=DEV)
    kvsel.gather_rows(src, idx, 7, 292, 8, dst)
    torch.cuda.synchronize()
    s, d = src.cpu().view(torch.int16), dst.cpu().view(torch.int16)
    want = O.gather_rows(s.numpy(), [5, 0, 299, 17, 17], 292, 8)
    assert np.array_equal(d[[0, 1, 2, 3, 4]].numpy(), want[:5])
    assert np.array_equal(d[7:].numpy(), want[5:])
    assert torch.all(d[5:7] == 0)    # out-of-range indices give zero rows


@pytest.mark.parametrize("cols,n_src,idx,tail_begin,n_tail", [
    (296, 50, [3, 49, -2, 50, 7, 7, 0], 45, 5),     # rows of 592 bytes (fewer pieces than threads)
    (8192, 20, [19, 0, 5], 17, 6),                  # 16 KiB rows (two passes), a tail running past the source
    (64, 0, [0, 1], 0, 3),                          # an empty source: every row zero
    (4096, 9, [8], 0, 0),                           # one row
])
def test_gather_rows_shapes(cols, n_src, idx, tail_begin, n_tail):
    kvsel = K()
    g = torch.Generator().manual_seed(cols + n_src)
    src = torch.randint(-(1 << 15), 1 << 15, (max(n_src, 1), cols), generator=g, dtype=torch.int16)
    src = src.view(torch.bfloat16).to(DEV)[:n_src]   # (an empty source still has a valid address)
    it = torch.tensor(idx, dtype=torch.int32, device=DEV)
    rows = len(idx) + n_tail
    dst = torch.full((rows, cols), 3.0, dtype=torch.bfloat16, device=DEV)
    log_case("gather-shapes", cols, n_src, len(idx), n_tail)
    if n_src:
        kvsel.gather_rows(src, it, len(idx), tail_begin, n_tail, dst)
    else:   # through the C entry point: a valid buffer that holds no source row
        buf = torch.zeros((1, cols), dtype=torch.bfloat16, device=DEV)
        st = kvsel.lib().kvsel_gather_rows(ctypes.c_void_p(buf.data_ptr()), cols * 2, 0, ctypes.c_void_p(it.data_ptr()),
                                           len(idx), tail_begin, n_tail, ctypes.c_void_p(dst.data_ptr()), None)
        assert st == 0
    torch.cuda.synchronize()
    s_np = src.cpu().view(torch.int16).numpy() if n_src else np.zeros((0, cols), np.int16)
    d_np = dst.cpu().view(torch.int16).numpy()
    want = np.zeros((rows, cols), np.int16)
    for j, r in enumerate(list(idx) + list(range(tail_begin, tail_begin + n_tail))):
        if 0 <= r < n_src:
            want[j] = s_np[r]
    assert np.array_equal(d_np, want)


def test_determinism():
    kvsel = K()
    rng = np.random.default_rng(5)
    lens = [3000, 2000, 2500]
    segs = [(0, 2500), (100, 1900), (0, 2500)]
    kv, _, _, _ = make_kv(rng, 3, 8, lens, segs)
    q = torch.randn((3, 16, 128), generator=torch.Generator().manual_seed(1)).to(torch.bfloat16).to(DEV)
    res = []
    for _ in range(2):
        out = torch.zeros((3, 16, 128), dtype=torch.float32, device=DEV)
        sc = torch.zeros((3, 8, 2500), dtype=torch.float32, device=DEV)
        kvsel.dense_attn(kv, q, 16, SCALE, out, seg_scores=sc)
        idx = torch.zeros((3, 8, 100), dtype=torch.int32, device=DEV)
        kvsel.topk(sc, 1800, 100, idx)
        o2 = torch.zeros_like(out)
        kvsel.gather_attn(kv, q, 16, SCALE, idx, 100, o2)
        torch.cuda.synchronize()
        res.append((out.cpu(), sc.cpu(), idx.cpu(), o2.cpu()))
    # scores and kept indices are bit-reproducible; the attention kernels hand
    # rows to waves on demand, so outputs may differ in rounding only
    (o_a, sc_a, i_a, s_a), (o_b, sc_b, i_b, s_b) = res
    assert torch.equal(sc_a, sc_b) and torch.equal(i_a, i_b)
    assert (o_a - o_b).abs().max().item() < 1e-5
    assert (s_a - s_b).abs().max().item() < 1e-5


@pytest.mark.parametrize("L", [5, 37, 100])
def test_fork_copy_on_write(L):
    """kvsel_fork on a partly filled last block: the child reads the parent's
    rows bit for bit through its own table; rows appended afterwards by
    either branch stay invisible to the other; attention through the child's
    table matches the oracle on the child's rows; reference counts."""
    kvsel = K()
    hkv, nb, maxb = 4, 24, 10
    pool = kvsel.BlockPool(nb)
    kp = torch.randn((nb, hkv, 16, 128), generator=torch.Generator().manual_seed(L)).to(torch.bfloat16).to(DEV)
    vp = torch.randn((nb, hkv, 16, 128), generator=torch.Generator().manual_seed(L + 1)).to(torch.bfloat16).to(DEV)
    parent = np.full(maxb, -1, dtype=np.int32)
    nblk = -(-(L + 7) // 16)
    parent[:nblk] = pool.alloc(nblk)[::-1]          # any order of physical blocks
    log_case("fork", L)
    child = pool.fork(parent, L, kp, vp)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(child[:L // 16], parent[:L // 16])
    fresh = child[L // 16]
    assert fresh not in parent and pool.refcount(fresh) == 1
    assert all(pool.refcount(b) == 2 for b in parent[:L // 16]) and pool.refcount(parent[L // 16]) == 1
    kc, vc = kp.cpu(), vp.cpu()
    for g in range(hkv):
        for pc in (kc, vc):
            np.testing.assert_array_equal(O.logical_rows(pc, child, g, L), O.logical_rows(pc, parent, g, L))
    # both branches append 7 rows after the fork point
    newp = torch.randn((hkv, 7, 128), generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    newc = torch.randn((hkv, 7, 128), generator=torch.Generator().manual_seed(2)).to(torch.bfloat16)
    child_t = child.copy()
    if (L + 6) // 16 > L // 16:
        child_t[(L + 6) // 16] = pool.alloc(1)[0]
    for j in range(7):
        pos = L + j
        kp[int(parent[pos // 16]), :, pos % 16, :] = newp[:, j].to(DEV)
        kp[int(child_t[pos // 16]), :, pos % 16, :] = newc[:, j].to(DEV)
        vp[int(child_t[pos // 16]), :, pos % 16, :] = newc[:, j].to(DEV)
    kc, vc = kp.cpu(), vp.cpu()
    for g in range(hkv):
        cl = O.logical_rows(kc, child_t, g, L + 7)
        pl = O.logical_rows(kc, parent, g, L + 7)
        np.testing.assert_array_equal(cl[:L], pl[:L])
        np.testing.assert_array_equal(cl[L:], O.widen(newc[g]))
        np.testing.assert_array_equal(pl[L:], O.widen(newp[g]))
    # attention through the child's table
    G, n = 2, L + 7
    kv = kvsel.KV(kp, vp, torch.from_numpy(child_t[None]).to(DEV), torch.tensor([n], dtype=torch.int32, device=DEV),
                  torch.zeros(1, dtype=torch.int32, device=DEV), torch.zeros(1, dtype=torch.int32, device=DEV),
                  max_seq_len=n, max_seg_len=0, min_seg_len=0)
    q = torch.randn((1, hkv * G, 128), generator=torch.Generator().manual_seed(3)).to(torch.bfloat16).to(DEV)
    out = torch.zeros((1, hkv * G, 128), dtype=torch.float32, device=DEV)
    kvsel.dense_attn(kv, q, hkv * G, SCALE, out)
    torch.cuda.synchronize()
    for g in range(hkv):
        ref, _ = O.dense_attention(O.widen(q.cpu()[0, g * G:(g + 1) * G]), O.logical_rows(kc, child_t, g, n),
                                   O.logical_rows(vc, child_t, g, n), SCALE)
        assert_attn(out[0, g * G:(g + 1) * G].cpu().numpy(), ref, f"child g{g}")


# (G, m, batch, lens, segments, k): the drafts are each sequence's last m rows;
# ragged tiles, k = 0, a segment reaching into the drafts (cut at n - m), m * G
# at one block of 32 query rows, and past it (2, 3 and 16 blocks of 32)
VERIFY_CASES = [(1, 1, 1, [1], [(0, 1)], 0), (2, 4, 2, [17, 300], [(3, 10), (0, 290)], 5),
                (4, 8, 1, [4000], [(10, 3900)], 200), (8, 4, 2, [700, 129], [(64, 600), (0, 100)], 33),
                (1, 32, 1, [96], [(0, 40)], 40), (2, 4, 1, [50], [(5, 50)], 30),
                (2, 4, 1, [8300], [(100, 8200)], 7900), (4, 2, 3, [33, 34, 35], [(1, 30), (2, 2), (0, 33)], 0),
                (3, 4, 2, [17, 300], [(3, 10), (0, 290)], 5), (5, 6, 1, [700], [(64, 600)], 33),
                (6, 2, 2, [50, 129], [(5, 50), (0, 100)], 20), (7, 4, 1, [400], [(10, 300)], 100),
                (8, 8, 2, [700, 129], [(64, 600), (0, 100)], 33), (3, 25, 1, [400], [(10, 300)], 60),
                (8, 64, 1, [900], [(0, 700)], 100)]


@pytest.mark.parametrize("G,m,batch,lens,segs,k", VERIFY_CASES)
def test_verify_attention(G, m, batch, lens, segs, k):
    kvsel = K()
    rng = np.random.default_rng(1000 + G * 37 + m)
    hkv = 2
    hq = hkv * G
    kv, kc, vc, table = make_kv(rng, batch, hkv, lens, segs)
    # the segment each sequence is cut to: it ends no later than n - m
    cut = [(min(s0, max(n - m, 0)), min(max(s1, min(s0, max(n - m, 0))), max(n - m, 0)))
           for (s0, s1), n in zip(segs, lens)]
    idx_np = np.full((batch, hkv, max(k, 1)), -1, dtype=np.int32)
    for b in range(batch):
        sl = segs[b][1] - segs[b][0]          # picks over the declared segment; those past the cut are dropped
        for g in range(hkv):
            pick = rng.choice(sl, size=min(k, sl), replace=False) if sl and k else np.array([], np.int64)
            idx_np[b, g, : len(pick)] = pick
    idx = torch.from_numpy(idx_np).to(DEV) if k else None
    q = torch.randn((batch, m, hq, 128), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).to(DEV)
    out = torch.full((batch, m, hq, 128), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((batch, m, hq), float("nan"), dtype=torch.float32, device=DEV)
    log_case("verify", G, m, lens, k)
    kvsel.verify_attn(kv, q, m, hq, SCALE, idx, k, out, lse)
    torch.cuda.synchronize()
    qc = q.cpu()
    for b in range(batch):
        s0, s1 = cut[b]
        for g in range(hkv):
            Kl = O.logical_rows(kc, table[b], g, lens[b])
            Vl = O.logical_rows(vc, table[b], g, lens[b])
            sel = idx_np[b, g][(idx_np[b, g] >= 0) & (idx_np[b, g] < s1 - s0)] if k else np.array([], np.int64)
            rows = O.kept_rows(sel, s0, s1, lens[b])
            qd = O.widen(qc[b, :, g * G:(g + 1) * G])
            ref, rl = O.verify_attention(qd, Kl, Vl, rows, lens[b], SCALE)
            for r in range(m):
                got = out[b, r, g * G:(g + 1) * G].cpu().numpy()
                assert_attn(got, ref[r], f"verify b{b} g{g} draft{r}")
                assert np.abs(lse[b, r, g * G:(g + 1) * G].cpu().numpy() - rl[r]).max() < 1e-4


# (G, hkv, lengths): packed ragged sequences, one row, an empty sequence,
# several 128-row blocks with a ragged tail, every group size
PREFILL_CASES = [(1, 2, [1]), (2, 2, [31, 100]), (4, 2, [257]), (8, 1, [130, 0, 3, 64]), (4, 8, [700]),
                 (1, 1, [129, 64]), (3, 2, [31, 100]), (5, 1, [257]), (6, 2, [129, 3]), (7, 1, [200])]


def _prefill_inputs(seed, lens, hq, hkv):
    g = torch.Generator().manual_seed(seed)
    total = sum(lens)
    q = torch.randn((total, hq, 128), generator=g).to(torch.bfloat16)
    k = torch.randn((total, hkv, 128), generator=g).to(torch.bfloat16)
    v = torch.randn((total, hkv, 128), generator=g).to(torch.bfloat16)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))
    return q, k, v, cu


@pytest.mark.parametrize("G,hkv,lens", PREFILL_CASES)
def test_prefill_attention(G, hkv, lens):
    kvsel = K()
    hq = hkv * G
    q, k, v, cu = _prefill_inputs(40 + G * 7 + len(lens), lens, hq, hkv)
    total = sum(lens)
    out = torch.full((total, hq, 128), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((total, hq), float("nan"), dtype=torch.float32, device=DEV)
    log_case("prefill", G, hkv, lens)
    kvsel.prefill_attn(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), max(lens), SCALE, out, lse)
    torch.cuda.synchronize()
    got, gl = out.cpu().numpy(), lse.cpu().numpy()
    for b, n in enumerate(lens):
        s0 = int(cu[b])
        if n == 0:
            continue
        ref, rl = O.causal_prefill(O.widen(q[s0:s0 + n]), O.widen(k[s0:s0 + n]), O.widen(v[s0:s0 + n]), SCALE)
        assert_attn(got[s0:s0 + n].reshape(n * hq, 128), ref, f"prefill b{b}")
        assert np.abs(gl[s0:s0 + n].reshape(-1) - rl).max() < 1e-4


def test_prefill_attention_propagated_tokens():
    """The later layers' attention after a TSP layer at 32768 tokens: 6554
    top-ranked tokens plus 8 window tokens, 32q/8kv; sampled rows (the first
    and last positions of every head, random ones) against the oracle."""
    kvsel = K()
    n, hq, hkv = 6562, 32, 8
    q, k, v, cu = _prefill_inputs(77, [n], hq, hkv)
    out = torch.empty((n, hq, 128), dtype=torch.float32, device=DEV)
    lse = torch.empty((n, hq), dtype=torch.float32, device=DEV)
    log_case("prefill-full", n, hq, hkv)
    kvsel.prefill_attn(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), n, SCALE, out, lse)
    torch.cuda.synchronize()
    rng = np.random.default_rng(78)
    rows = [(0, h) for h in range(0, hq, 5)] + [(n - 1, h) for h in range(hq)] + \
        [(int(i), int(h)) for i, h in zip(rng.integers(0, n, 24), rng.integers(0, hq, 24))] + [(127, 3), (128, 4)]
    ref, rl = O.causal_prefill(O.widen(q), O.widen(k), O.widen(v), SCALE, rows=rows)
    got = out.cpu().numpy()
    gl = lse.cpu().numpy()
    assert_attn(np.stack([got[i, h] for i, h in rows]), ref, "prefill full")
    assert np.abs(np.array([gl[i, h] for i, h in rows]) - rl).max() < 1e-4


# V magnitudes that the fp16 staging of the prefill and shared-range kernels
# must carry: beyond the fp16 range everywhere, far below it (fp16
# subnormals), a few huge rows among ordinary ones, and a ramp from 2^-40 to
# beyond fp16 along the first axis (the scale grows tile after tile).  Powers
# of two keep the bf16 values exact.
WIDE_V = ("huge", "tiny", "mixed", "ramp")


def widen_v(v, kind, seed, ramp_step=1.0):
    """v (bf16) with the vectors along its last axis scaled as kind says
    (ramp: by 2^(floor(i * ramp_step) - 40) at index i of the first axis)."""
    x = v.detach().cpu().float()
    if kind == "huge":
        x *= 2.0 ** 17
    elif kind == "tiny":
        x *= 2.0 ** -40
    elif kind == "mixed":
        pick = torch.rand(v.shape[:-1], generator=torch.Generator().manual_seed(seed)) < 0.05
        x[pick] *= 2.0 ** 20
    else:
        e = np.minimum(np.floor(np.arange(x.shape[0]) * ramp_step) - 40, 60)
        x *= torch.from_numpy(np.exp2(e)).float().view(-1, *([1] * (x.dim() - 1)))
    return x.to(torch.bfloat16).to(v.device)


def assert_attn_scaled(got, ref, vmax, what=""):
    """The attention acceptance test with the absolute bound taken relative
    to the largest |V| (the relative L2 bound is scale-free)."""
    return assert_attn(np.asarray(got, dtype=np.float64) / vmax, np.asarray(ref, dtype=np.float64) / vmax, what)


@pytest.mark.parametrize("kind", WIDE_V)
def test_prefill_attention_wide_v(kind):
    """Causal prefill with V beyond, far below, partly far beyond the fp16
    range, or ramping across it, against the oracle (each query row's errors
    relative to the largest |V| it sees)."""
    kvsel = K()
    G, hkv, lens = 2, 2, [300, 1, 77, 130]
    hq = hkv * G
    q, k, v, cu = _prefill_inputs(61, lens, hq, hkv)
    v = widen_v(v, kind, 62, ramp_step=1 / 8)
    total = sum(lens)
    out = torch.full((total, hq, 128), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((total, hq), float("nan"), dtype=torch.float32, device=DEV)
    log_case("prefill-wide-v", kind, lens)
    kvsel.prefill_attn(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), max(lens), SCALE, out, lse)
    torch.cuda.synchronize()
    got, gl = out.cpu().numpy(), lse.cpu().numpy()
    for b, n in enumerate(lens):
        s0 = int(cu[b])
        ref, rl = O.causal_prefill(O.widen(q[s0:s0 + n]), O.widen(k[s0:s0 + n]), O.widen(v[s0:s0 + n]), SCALE)
        seen = np.maximum.accumulate(v[s0:s0 + n].float().abs().amax(dim=(1, 2)).numpy().astype(np.float64))
        sc = np.repeat(seen, hq)[:, None]                    # rows position-major, like ref
        assert_attn(got[s0:s0 + n].reshape(n * hq, 128) / sc, ref / sc, f"prefill {kind} b{b}")
        assert np.abs(gl[s0:s0 + n].reshape(-1) - rl).max() < 1e-4


def _shared_prefix_kv(rng, batch, hkv, prefix_len, suffix_max):
    """A paged cache whose sequences share their first prefix_len rows (the
    same blocks, placed at random), each with a private suffix."""
    from synth.gen import shared_prefix_table
    kvsel = K()
    pb = -(-prefix_len // 16)
    suffix = rng.integers(1, suffix_max + 1, size=batch)
    table, nb = shared_prefix_table(pb, -(-suffix // 16))
    perm = rng.permutation(nb + 2).astype(np.int32)    # scatter the blocks over a slightly larger pool
    table = perm[table]
    g = torch.Generator().manual_seed(int(rng.integers(1 << 30)))
    kp = torch.randn((nb + 2, hkv, 16, 128), generator=g).to(torch.bfloat16).to(DEV)
    vp = torch.randn((nb + 2, hkv, 16, 128), generator=g).to(torch.bfloat16).to(DEV)
    lens = (pb * 16 + suffix).astype(np.int32)
    zeros = torch.zeros(batch, dtype=torch.int32, device=DEV)
    kv = kvsel.KV(kp, vp, torch.from_numpy(table).to(DEV), torch.from_numpy(lens).to(DEV), zeros, zeros,
                  max_seq_len=int(lens.max()), max_seg_len=0, min_seg_len=0, shared_rows=prefix_len)
    return kv, cpu_pool(kp), cpu_pool(vp), table, lens


# (G, batch, prefix rows, [row_begin, row_end), parts): ranges not on block
# edges, several 128-row query blocks with a ragged last one, an empty range,
# parts of the range (some empty)
SHARED_CASES = [(2, 5, 160, (37, 160), 1, 1), (1, 3, 64, (0, 64), 1, 1), (4, 70, 1024, (300, 1024), 4, 1),
                (8, 20, 96, (5, 90), 3, 1), (2, 9, 48, (10, 10), 1, 1), (2, 600, 256, (64, 250), 2, 1),
                (1, 4, 128, (0, 100), 5, 1), (2, 30, 200, (16, 180), 2, 3),
                (3, 7, 160, (37, 160), 2, 1), (6, 9, 200, (16, 180), 1, 2), (5, 40, 96, (5, 90), 3, 1),
                (7, 3, 64, (0, 64), 1, 4),
                # ranges touching the most cache blocks a call takes (1024), on and off block edges
                (2, 6, 16384, (0, 16384), 3, 1), (2, 6, 16400, (1, 16384), 2, 1)]


@pytest.mark.parametrize("G,batch,prefix,rng_rows,splits,qps", SHARED_CASES)
def test_shared_attention(G, batch, prefix, rng_rows, splits, qps):
    kvsel = K()
    rng = np.random.default_rng(3000 + G * 11 + batch)
    hkv = 2
    hq = hkv * G
    kv, kc, vc, table, lens = _shared_prefix_kv(rng, batch, hkv, prefix, 40)
    q = torch.randn((batch, qps, hq, 128), generator=torch.Generator().manual_seed(9)).to(torch.bfloat16).to(DEV)
    parts = torch.full((splits, batch, qps, hq, 128), float("nan"), dtype=torch.float32, device=DEV)
    plse = torch.full((splits, batch, qps, hq), float("nan"), dtype=torch.float32, device=DEV)
    rb, re = rng_rows
    log_case("shared", G, batch, prefix, rb, re, splits, qps)
    kvsel.shared_attn(kv, q, hq, SCALE, rb, re, parts, plse, splits=splits, q_per_seq=qps)
    out = torch.empty((batch, qps, hq, 128), dtype=torch.float32, device=DEV)
    lse = torch.empty((batch, qps, hq), dtype=torch.float32, device=DEV)
    kvsel.merge_attn(parts, plse, out, lse)
    torch.cuda.synchronize()
    assert not torch.isnan(parts).any() and not torch.isnan(plse).any()   # every part written
    qc = q.cpu()
    check = [(b, r) for b in range(batch) for r in range(qps)]
    if len(check) > 20:
        check = [check[i] for i in rng.choice(len(check), size=20, replace=False)]
    for b, r in check:
        for g in range(hkv):
            got = out[b, r, g * G:(g + 1) * G].cpu().numpy()
            gl = lse[b, r, g * G:(g + 1) * G].cpu().numpy()
            if re == rb:
                assert np.all(got == 0) and np.all(np.isneginf(gl))
                continue
            Kl = O.logical_rows(kc, table[b], g, int(lens[b]))
            Vl = O.logical_rows(vc, table[b], g, int(lens[b]))
            ref, rl = O.attention(O.widen(qc[b, r, g * G:(g + 1) * G]), Kl, Vl, np.arange(rb, re), SCALE)
            assert_attn(got, ref, f"shared b{b} q{r} g{g}")
            assert np.abs(gl - rl).max() < 1e-4


@pytest.mark.parametrize("kind", WIDE_V)
def test_shared_attention_wide_v(kind):
    """The shared-range kernel with the range's V beyond, far below, or partly
    far beyond the fp16 range: parts and the folded (accumulate) form against
    the oracle, errors relative to the largest |V|."""
    import dataclasses
    kvsel = K()
    rng = np.random.default_rng(3500)
    G, batch, hkv, prefix, qps = 2, 40, 2, 400, 2
    hq = hkv * G
    kv, kc, vc, table, lens = _shared_prefix_kv(rng, batch, hkv, prefix, 30)
    vp = widen_v(kv.v_pool, kind, 3501, ramp_step=2.0)
    kv = dataclasses.replace(kv, v_pool=vp)
    vc = cpu_pool(vp)
    rb, re = 21, 390
    vmax = max(float(np.abs(O.logical_rows(vc, table[0], g, re)[rb:]).max()) for g in range(hkv))
    q = torch.randn((batch, qps, hq, 128), generator=torch.Generator().manual_seed(17)).to(torch.bfloat16).to(DEV)
    parts = torch.empty((3, batch, qps, hq, 128), dtype=torch.float32, device=DEV)
    plse = torch.empty((3, batch, qps, hq), dtype=torch.float32, device=DEV)
    log_case("shared-wide-v", kind)
    kvsel.shared_attn(kv, q, hq, SCALE, rb, re, parts, plse, splits=3, q_per_seq=qps)
    out = torch.empty((batch, qps, hq, 128), dtype=torch.float32, device=DEV)
    lse = torch.empty((batch, qps, hq), dtype=torch.float32, device=DEV)
    kvsel.merge_attn(parts, plse, out, lse)
    # folded: an empty other part (lse -inf) leaves the range's own attention
    acc_o = torch.zeros((batch, qps, hq, 128), dtype=torch.float32, device=DEV)
    acc_l = torch.full((batch, qps, hq), float("-inf"), dtype=torch.float32, device=DEV)
    kvsel.shared_attn(kv, q, hq, SCALE, rb, re, acc_o, acc_l, splits=1, q_per_seq=qps, accumulate=True)
    torch.cuda.synchronize()
    qc = q.cpu()
    for b in rng.choice(batch, size=8, replace=False):
        for r in range(qps):
            for g in range(hkv):
                Kl = O.logical_rows(kc, table[b], g, int(lens[b]))
                Vl = O.logical_rows(vc, table[b], g, int(lens[b]))
                ref, rl = O.attention(O.widen(qc[b, r, g * G:(g + 1) * G]), Kl, Vl, np.arange(rb, re), SCALE)
                for name, o, l in (("parts", out, lse), ("accumulate", acc_o, acc_l)):
                    assert_attn_scaled(o[b, r, g * G:(g + 1) * G].cpu().numpy(), ref, vmax,
                                       f"shared {kind} {name} b{b} q{r} g{g}")
                    assert np.abs(l[b, r, g * G:(g + 1) * G].cpu().numpy() - rl).max() < 1e-4


def test_shared_attention_logits_stay_in_their_row():
    """A device segment longer than ld_logits (a bad value) writes at most
    ld_logits entries: the guard past the logits buffer stays NaN, and the
    row's first ld_logits entries are its dots."""
    import dataclasses
    kvsel = K()
    rng = np.random.default_rng(3400)
    G, batch, hkv, prefix = 2, 6, 2, 160
    hq = hkv * G
    kv, kc, vc, table, lens = _shared_prefix_kv(rng, batch, hkv, prefix, 20)
    s0, s1, ld = 4, 100, 96
    seg_e = np.full(batch, s1, dtype=np.int32)
    seg_e[-1] = 150                                   # longer than max_seg_len = ld
    kv = dataclasses.replace(kv, seg_begin=torch.full((batch,), s0, dtype=torch.int32, device=DEV),
                             seg_end=torch.from_numpy(seg_e).to(DEV), max_seg_len=s1 - s0, min_seg_len=s1 - s0)
    q = torch.randn((batch, hq, 128), generator=torch.Generator().manual_seed(7)).to(torch.bfloat16).to(DEV)
    parts = torch.empty((2, batch, hq, 128), dtype=torch.float32, device=DEV)
    plse = torch.empty((2, batch, hq), dtype=torch.float32, device=DEV)
    buf = torch.full((batch * hq * ld + 256,), float("nan"), dtype=torch.float32, device=DEV)
    logits = buf[:batch * hq * ld].view(batch, hq, ld)
    log_case("shared-logits-clamp", batch, ld)
    kvsel.shared_attn(kv, q, hq, SCALE, 0, prefix, parts, plse, splits=2, logits=logits)
    torch.cuda.synchronize()
    assert torch.all(torch.isnan(buf[batch * hq * ld:]))
    b = batch - 1
    lg, qc = logits.cpu().numpy(), q.cpu()
    for g in range(hkv):
        Kl = O.logical_rows(kc, table[b], g, int(lens[b]))
        ref = O.logits(O.widen(qc[b, g * G:(g + 1) * G]), Kl[s0:s0 + ld], 1.0)
        assert np.abs(lg[b, g * G:(g + 1) * G] - ref).max() <= 1e-5 * max(1.0, np.abs(ref).max())


@pytest.mark.parametrize("G,batch,prefix,rng_rows,qps", [(2, 5, 160, (37, 160), 1), (4, 70, 1024, (300, 1024), 1),
                                                      (2, 9, 48, (10, 10), 1), (2, 30, 200, (16, 180), 3),
                                                      (1, 300, 64, (0, 64), 2)])
def test_shared_attention_accumulate(G, batch, prefix, rng_rows, qps):
    """accumulate = 1: out/lse hold another part on entry (random values,
    some rows empty: lse = -inf); the call leaves the exact merge of that part
    and the range, against the oracle's merge of the two."""
    kvsel = K()
    rng = np.random.default_rng(3300 + G * 7 + batch)
    hkv = 2
    hq = hkv * G
    kv, kc, vc, table, lens = _shared_prefix_kv(rng, batch, hkv, prefix, 40)
    q = torch.randn((batch, qps, hq, 128), generator=torch.Generator().manual_seed(13)).to(torch.bfloat16).to(DEV)
    g = torch.Generator().manual_seed(batch + qps)
    o_in = torch.randn((batch, qps, hq, 128), generator=g)
    l_in = torch.randn((batch, qps, hq), generator=g) * 3
    l_in.view(-1)[::5] = float("-inf")           # rows whose other part is empty
    out, lse = o_in.to(DEV), l_in.to(DEV)
    rb, re = rng_rows
    log_case("shared-acc", G, batch, prefix, rb, re, qps)
    kvsel.shared_attn(kv, q, hq, SCALE, rb, re, out, lse, splits=1, q_per_seq=qps, accumulate=True)
    torch.cuda.synchronize()
    qc = q.cpu()
    got_o, got_l = out.cpu().numpy(), lse.cpu().numpy()
    check = [(b, r) for b in range(batch) for r in range(qps)]
    if len(check) > 24:
        check = [check[i] for i in rng.choice(len(check), size=24, replace=False)]
    for b, r in check:
        for gi in range(hkv):
            hs = slice(gi * G, (gi + 1) * G)
            if re > rb:
                Kl = O.logical_rows(kc, table[b], gi, int(lens[b]))
                Vl = O.logical_rows(vc, table[b], gi, int(lens[b]))
                so, sl = O.attention(O.widen(qc[b, r, hs]), Kl, Vl, np.arange(rb, re), SCALE)
            else:
                so, sl = np.zeros((G, 128)), np.full(G, -np.inf)
            ref, rl = O.merge_attention(o_in[b, r, hs].numpy().astype(np.float64),
                                        l_in[b, r, hs].numpy().astype(np.float64), so, sl)
            assert_attn(got_o[b, r, hs], ref, f"shared-acc b{b} q{r} g{gi}")
            fin = np.isfinite(rl)
            assert np.abs(got_l[b, r, hs][fin] - rl[fin]).max(initial=0) < 1e-4
            assert np.all(np.isneginf(got_l[b, r, hs][~fin])) and np.all(got_o[b, r, hs][~fin] == 0)


def test_shared_attention_accumulate_with_logits():
    """One call that both folds the range into an existing output (accumulate)
    and writes the segment logits -- a focal layer whose prefix is one part."""
    import dataclasses
    kvsel = K()
    rng = np.random.default_rng(3500)
    G, batch, hkv, prefix = 2, 21, 2, 176
    hq = hkv * G
    kv, kc, vc, table, lens = _shared_prefix_kv(rng, batch, hkv, prefix, 25)
    s0, s1 = 0, 150
    kv = dataclasses.replace(kv, seg_begin=torch.full((batch,), s0, dtype=torch.int32, device=DEV),
                             seg_end=torch.full((batch,), s1, dtype=torch.int32, device=DEV),
                             max_seg_len=s1 - s0, min_seg_len=s1 - s0)
    q = torch.randn((batch, hq, 128), generator=torch.Generator().manual_seed(3)).to(torch.bfloat16).to(DEV)
    g = torch.Generator().manual_seed(33)
    o_in = torch.randn((batch, hq, 128), generator=g)
    l_in = torch.randn((batch, hq), generator=g) * 2
    out, lse = o_in.to(DEV), l_in.to(DEV)
    logits = torch.full((batch, hq, s1 - s0), float("nan"), dtype=torch.float32, device=DEV)
    log_case("shared-acc-logits", batch, prefix)
    kvsel.shared_attn(kv, q, hq, SCALE, 0, prefix, out, lse, splits=1, logits=logits, accumulate=True)
    torch.cuda.synchronize()
    qc, lg = q.cpu(), logits.cpu().numpy()
    for b in range(0, batch, 3):
        for gi in range(hkv):
            hs = slice(gi * G, (gi + 1) * G)
            Kl = O.logical_rows(kc, table[b], gi, int(lens[b]))
            Vl = O.logical_rows(vc, table[b], gi, int(lens[b]))
            qg = O.widen(qc[b, hs])
            so, sl = O.attention(qg, Kl, Vl, np.arange(0, prefix), SCALE)
            ref, rl = O.merge_attention(o_in[b, hs].numpy().astype(np.float64), l_in[b, hs].numpy().astype(np.float64),
                                        so, sl)
            assert_attn(out[b, hs].cpu().numpy(), ref, f"acc+logits b{b} g{gi}")
            assert np.abs(lse[b, hs].cpu().numpy() - rl).max() < 1e-4
            ref_l = O.logits(qg, Kl[s0:s1], 1.0)
            assert np.abs(lg[b, hs] - ref_l).max() <= 1e-5 * max(1.0, np.abs(ref_l).max())


@pytest.mark.parametrize("splits", [1, 3])
def test_shared_attention_skips_unattended_rows(splits):
    """Rows the kernel reads but must not attend hold NaN: every pool row
    outside [row_begin, row_end) (rows before row_begin in its first block,
    the unused rows of the last shared block, the spare blocks, the suffixes),
    and one block inside the range is not a pool block (-1 in every table):
    its rows are skipped and their logits are -inf.  Output and lse against
    the oracle over the remaining rows."""
    import dataclasses
    kvsel = K()
    rng = np.random.default_rng(3200 + splits)
    G, batch, hkv, prefix = 2, 33, 2, 200
    hq = hkv * G
    kv, kc, vc, table, lens = _shared_prefix_kv(rng, batch, hkv, prefix, 30)
    rb, re, hole = 21, 200, 5                    # block 5 of the range: rows 80 .. 95
    keep = np.zeros(kv.k_pool.shape[:2] + (16,), dtype=bool)   # [block][kv head][row]
    for j in range(rb, re):
        keep[table[0][j // 16], :, j % 16] = True
    nan_rows = torch.from_numpy(~keep).to(DEV)
    kv.k_pool[nan_rows] = float("nan")
    kv.v_pool[nan_rows] = float("nan")
    holed = table.copy()
    holed[:, hole] = -1
    s0, s1 = 4, 150
    kvh = dataclasses.replace(kv, block_table=torch.from_numpy(holed).to(DEV),
                              seg_begin=torch.full((batch,), s0, dtype=torch.int32, device=DEV),
                              seg_end=torch.full((batch,), s1, dtype=torch.int32, device=DEV),
                              max_seg_len=s1 - s0, min_seg_len=s1 - s0)
    q = torch.randn((batch, hq, 128), generator=torch.Generator().manual_seed(11)).to(torch.bfloat16).to(DEV)
    parts = torch.empty((splits, batch, hq, 128), dtype=torch.float32, device=DEV)
    plse = torch.empty((splits, batch, hq), dtype=torch.float32, device=DEV)
    logits = torch.full((batch, hq, 160), float("nan"), dtype=torch.float32, device=DEV)
    log_case("shared-skips", splits, batch, rb, re, hole)
    kvsel.shared_attn(kvh, q, hq, SCALE, rb, re, parts, plse, splits=splits, logits=logits)
    out = torch.empty((batch, hq, 128), dtype=torch.float32, device=DEV)
    lse = torch.empty((batch, hq), dtype=torch.float32, device=DEV)
    kvsel.merge_attn(parts, plse, out, lse)
    torch.cuda.synchronize()
    rows = np.array([j for j in range(rb, re) if j // 16 != hole])
    qc, lg = q.cpu(), logits.cpu().numpy()
    for b in range(0, batch, 4):
        for g in range(hkv):
            Kl = O.logical_rows(kc, table[b], g, int(lens[b]))
            Vl = O.logical_rows(vc, table[b], g, int(lens[b]))
            qg = O.widen(qc[b, g * G:(g + 1) * G])
            ref, rl = O.attention(qg, Kl, Vl, rows, SCALE)
            assert_attn(out[b, g * G:(g + 1) * G].cpu().numpy(), ref, f"shared-skips b{b} g{g}")
            assert np.abs(lse[b, g * G:(g + 1) * G].cpu().numpy() - rl).max() < 1e-4
            got = lg[b, g * G:(g + 1) * G]
            assert np.all(np.isnan(got[:, :rb - s0]))              # segment rows before the range: untouched
            inside = np.array([j for j in range(rb, s1) if j // 16 != hole])
            ref_l = O.logits(qg, Kl[inside], 1.0)
            assert np.abs(got[:, inside - s0] - ref_l).max() <= 1e-5 * max(1.0, np.abs(ref_l).max())
            assert np.all(np.isneginf(got[:, 16 * hole - s0:16 * hole + 16 - s0]))
            assert np.all(np.isnan(got[:, s1 - s0:]))               # past the segment: untouched


@pytest.mark.parametrize("rows,parts,inplace", [(1, 2, False), (37, 2, False), (1000, 2, True), (300, 5, True),
                                                (9, 1, False)])
def test_merge_attention(rows, parts, inplace):
    """N parts against the oracle's pairwise merges folded left."""
    kvsel = K()
    g = torch.Generator().manual_seed(rows + parts)
    o = torch.randn((parts, rows, 128), generator=g)
    ls = torch.randn((parts, rows), generator=g) * 3
    for p in range(parts):
        ls[p, p::7] = float("-inf")    # some rows with empty parts
    ls[:, 0] = float("-inf")           # a row with every part empty
    ref, rl = np.zeros((rows, 128)), np.full(rows, -np.inf)   # the empty set, then every part merged in
    for p in range(parts):
        ref, rl = O.merge_attention(ref, rl, o[p].numpy(), ls[p].numpy())
    do, dl = o.to(DEV), ls.to(DEV)
    out, lse = (do[parts - 1], dl[parts - 1]) if inplace else (torch.empty_like(do[0]), torch.empty_like(dl[0]))
    log_case("merge", rows, parts, inplace)
    kvsel.merge_attn(do, dl, out, lse)
    torch.cuda.synchronize()
    got, gl = out.cpu().numpy(), lse.cpu().numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-5)
    fin = np.isfinite(rl)
    np.testing.assert_allclose(gl[fin], rl[fin], rtol=1e-6, atol=1e-5)
    assert np.all(np.isneginf(gl[~fin])) and np.all(got[~fin] == 0)


def test_shared_attention_segment_logits():
    """The raw dots the shared-rows kernel writes for the segment rows inside
    its range (three parts), against the oracle's logits; entries past the
    range stay untouched."""
    kvsel = K()
    rng = np.random.default_rng(3100)
    G, batch, hkv, prefix = 2, 40, 2, 160
    hq = hkv * G
    kv, kc, vc, table, lens = _shared_prefix_kv(rng, batch, hkv, prefix, 30)
    s0, s1 = 4, 100
    seg_b = torch.full((batch,), s0, dtype=torch.int32, device=DEV)
    seg_e = torch.full((batch,), s1, dtype=torch.int32, device=DEV)
    import dataclasses
    kv = dataclasses.replace(kv, seg_begin=seg_b, seg_end=seg_e, max_seg_len=s1 - s0, min_seg_len=s1 - s0)
    q = torch.randn((batch, hq, 128), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).to(DEV)
    parts = torch.empty((3, batch, hq, 128), dtype=torch.float32, device=DEV)
    plse = torch.empty((3, batch, hq), dtype=torch.float32, device=DEV)
    ld = 128
    logits = torch.full((batch, hq, ld), float("nan"), dtype=torch.float32, device=DEV)
    log_case("shared-logits", batch, s0, s1)
    kvsel.shared_attn(kv, q, hq, SCALE, 0, 90, parts, plse, splits=3, logits=logits)   # the range ends inside the segment
    torch.cuda.synchronize()
    lg, qc = logits.cpu().numpy(), q.cpu()
    for b in range(0, batch, 7):
        for g in range(hkv):
            Kl = O.logical_rows(kc, table[b], g, int(lens[b]))
            ref = O.logits(O.widen(qc[b, g * G:(g + 1) * G]), Kl[s0:90], 1.0)
            got = lg[b, g * G:(g + 1) * G, :90 - s0]
            assert np.abs(got - ref).max() <= 1e-5 * max(1.0, np.abs(ref).max())
            assert np.all(np.isnan(lg[b, g * G:(g + 1) * G, 90 - s0:]))


def _holed_reference(kc, vc, table_row, g, qg, n, s0, s1, hole):
    """Oracle view of a sequence whose cache block `hole` is missing: its rows
    are not attended (softmax over the remaining rows) and score 0."""
    Kl = O.logical_rows(kc, table_row, g, n)
    Vl = O.logical_rows(vc, table_row, g, n)
    rows = np.array([j for j in range(n) if j // 16 != hole])
    seg_rows = np.array([j for j in range(s0, s1) if j // 16 != hole])
    sc = np.zeros(s1 - s0)
    sc[seg_rows - s0] = O.focal_scores(qg, Kl[seg_rows], 0, len(seg_rows), SCALE)
    out, _ = O.attention(qg, Kl, Vl, rows, SCALE)
    return sc, out


@pytest.mark.parametrize("form", ["fused", "split", "score"])
def test_focal_selection_skips_missing_block(form):
    """A segment block that is not a pool block (-1 in the table) is skipped:
    its rows get logit -inf, probability 0 and score 0, and the rest of the
    segment is normalised without them.  fused: the one-kernel focal pass
    (256 pairs); split: split attention with the logits in the workspace and
    the standalone selection; score: kvsel_score's logits kernel and
    normaliser, then kvsel_topk.  The workspace is filled with NaN first, so a
    logit that is not written would show."""
    import dataclasses
    kvsel = K()
    rng = np.random.default_rng(4400 + len(form))
    G = 2
    batch, hkv = (32, 8) if form == "fused" else (3, 4)
    hq = hkv * G
    n, s0, s1, hole = 700, 20, 600, 9          # block 9: rows 144 .. 159, inside the segment
    k = 40
    lens = [n] * batch
    kv, kc, vc, table = make_kv(rng, batch, hkv, lens, [(s0, s1)] * batch)
    holed = table.copy()
    holed[:, hole] = -1
    kvh = dataclasses.replace(kv, block_table=torch.from_numpy(holed).to(DEV))
    ws = kvsel.Workspace(DEV, 1 << 22)
    ws.buf.fill_(0xFF)                          # NaN in every float slot
    ws.buf[:65536].zero_()                      # the reserved head stays zero
    q = torch.randn((batch, hq, 128), generator=torch.Generator().manual_seed(44)).to(torch.bfloat16).to(DEV)
    out = torch.zeros((batch, hq, 128), dtype=torch.float32, device=DEV)
    sc = torch.full((batch, hkv, s1 - s0), float("nan"), dtype=torch.float32, device=DEV)
    idx = torch.zeros((batch, hkv, k), dtype=torch.int32, device=DEV)
    log_case("missing-block", form, batch, hkv)
    if form == "score":
        kvsel.score(kvh, q.view(batch, 1, hq, 128), 1, hq, SCALE, 0, 0, True, 1, sc, ws=ws)
        kvsel.topk(sc, s1 - s0, k, idx)
    else:
        kvsel.focal_attn(kvh, q, hq, SCALE, out, k, idx, seg_scores=sc, ws=ws)
    torch.cuda.synchronize()
    qc = q.cpu()
    for b in range(0, batch, max(1, batch // 4)):
        for g in range(hkv):
            qg = O.widen(qc[b, g * G:(g + 1) * G])
            ref_s, ref_o = _holed_reference(kc, vc, table[b], g, qg, n, s0, s1, hole)
            got = sc[b, g].cpu().numpy()
            assert np.all(got[16 * hole - s0:16 * hole + 16 - s0] == 0.0), (form, b, g)
            kept = (np.arange(s0, s1) // 16) != hole    # segment rows outside the missing block
            assert rel_err(got[kept], ref_s[kept]) < 2e-6, (form, b, g)
            ok, nd = O.tie_band_check(idx[b, g].cpu().numpy(), ref_s, k, BAND)
            assert ok, (form, b, g, nd)
            if form != "score":
                assert_attn(out[b, g * G:(g + 1) * G].cpu().numpy(), ref_o, f"missing-block out b{b} g{g}")


def test_select_logits_skips_missing_block():
    """The shared-prefix cascade's selection with one block of the shared
    range missing from every table: kvsel_shared_attn writes -inf logits for
    its rows, and kvsel_select_logits gives them score 0 and normalises the
    segment over the remaining rows (against the oracle's focal scores and
    top-k over those rows)."""
    import dataclasses
    kvsel = K()
    rng = np.random.default_rng(4500)
    G, batch, hkv, prefix = 2, 33, 2, 200
    hq = hkv * G
    kv, kc, vc, table, lens = _shared_prefix_kv(rng, batch, hkv, prefix, 30)
    rb, re, hole = 16, 200, 5                    # block 5 of the range: rows 80 .. 95
    s0, s1 = 32, 150
    k = 12
    holed = table.copy()
    holed[:, hole] = -1
    kvh = dataclasses.replace(kv, block_table=torch.from_numpy(holed).to(DEV),
                              seg_begin=torch.full((batch,), s0, dtype=torch.int32, device=DEV),
                              seg_end=torch.full((batch,), s1, dtype=torch.int32, device=DEV),
                              max_seg_len=s1 - s0, min_seg_len=s1 - s0)
    q = torch.randn((batch, hq, 128), generator=torch.Generator().manual_seed(45)).to(torch.bfloat16).to(DEV)
    parts = torch.empty((1, batch, hq, 128), dtype=torch.float32, device=DEV)
    plse = torch.empty((1, batch, hq), dtype=torch.float32, device=DEV)
    logits = torch.full((batch, hq, s1 - s0), float("nan"), dtype=torch.float32, device=DEV)
    sc = torch.full((batch, hkv, s1 - s0), float("nan"), dtype=torch.float32, device=DEV)
    idx = torch.zeros((batch, hkv, k), dtype=torch.int32, device=DEV)
    log_case("select-logits-missing-block", batch, rb, re, hole)
    kvsel.shared_attn(kvh, q, hq, SCALE, rb, re, parts, plse, splits=1, logits=logits)
    kvsel.select_logits(kvh, logits, hq, SCALE, k, idx, seg_scores=sc)
    torch.cuda.synchronize()
    qc = q.cpu()
    seg_rows = np.array([j for j in range(s0, s1) if j // 16 != hole])
    for b in range(0, batch, 4):
        for g in range(hkv):
            Kl = O.logical_rows(kc, table[b], g, int(lens[b]))
            qg = O.widen(qc[b, g * G:(g + 1) * G])
            ref = np.zeros(s1 - s0)
            ref[seg_rows - s0] = O.focal_scores(qg, Kl[seg_rows], 0, len(seg_rows), SCALE)
            got = sc[b, g].cpu().numpy()
            assert np.all(got[16 * hole - s0:16 * hole + 16 - s0] == 0.0), (b, g)
            assert rel_err(got[seg_rows - s0], ref[seg_rows - s0]) < 2e-6, (b, g)
            ok, nd = O.tie_band_check(idx[b, g].cpu().numpy(), ref, k, BAND)
            assert ok, (b, g, nd)


@pytest.mark.parametrize("G,n", [(1, 3000), (2, 3000), (4, 3000), (2, 8300)])
def test_split_count_invariance(G, n):
    """The same two sequences attended alone (few pairs: each pair's rows split
    over many work-groups, the records merged by the last of them) and
    replicated into a launch of 256+ (sequence, kv head) pairs (about one
    work-group per pair): the outputs agree up to summation order, with each
    other and with the oracle, for gathered and dense attention; with
    KVSEL_FLAG_DETERMINISTIC the replicas of one sequence are equal bit for
    bit.  A missing barrier in the row hand-out, the wave merge or the record
    merge would show as a difference between the split counts or between the
    replicas.  n = 8300: more rows per pair than one work-group's row table
    holds, so even the replicated dense launch splits each pair in two."""
    kvsel = K()
    rng = np.random.default_rng(4400 + G + n)
    hkv, seg, k = 2, (100, n - 900), 150
    hq = hkv * G
    kp, vp, table = random_paged(rng, 2, hkv, n, DEV)
    idx_np = np.stack([np.stack([np.sort(rng.choice(seg[1] - seg[0], size=k, replace=False)) for _ in range(hkv)])
                       for _ in range(2)]).astype(np.int32)
    q = torch.randn((2, hq, 128), generator=torch.Generator().manual_seed(11)).to(torch.bfloat16).to(DEV)
    reps = 256 // (2 * hkv) + 1
    i32 = lambda x: torch.as_tensor(np.asarray(x, dtype=np.int32)).to(DEV)

    def run(R, det):
        b = 2 * R
        kv = kvsel.KV(kp, vp, i32(np.tile(table, (R, 1))), i32([n] * b), i32([seg[0]] * b), i32([seg[1]] * b),
                      max_seq_len=n, max_seg_len=seg[1] - seg[0], min_seg_len=seg[1] - seg[0], deterministic=det)
        qq = q.repeat(R, 1, 1).contiguous()
        idx = i32(np.tile(idx_np, (R, 1, 1)))
        og = torch.zeros((b, hq, 128), dtype=torch.float32, device=DEV)
        lg = torch.zeros((b, hq), dtype=torch.float32, device=DEV)
        od = torch.zeros_like(og)
        ld = torch.zeros_like(lg)
        kvsel.gather_attn(kv, qq, hq, SCALE, idx, k, og, lg)
        kvsel.dense_attn(kv, qq, hq, SCALE, od, ld)
        torch.cuda.synchronize()
        return [x.cpu().numpy().reshape(R, 2, *x.shape[1:]) for x in (og, lg, od, ld)]

    log_case("split invariance", G, reps)
    small = run(1, False)
    big = run(reps, False)
    for a, bb in zip(small, big):
        scale_ = max(float(np.abs(a).max()), 1.0)
        assert float(np.abs(bb - a).max()) <= 1e-5 * scale_
    det = run(reps, True)
    for x in det:
        assert all(np.array_equal(x[r], x[0]) for r in range(reps)), "deterministic replicas differ"
    kc, vc, qc = cpu_pool(kp), cpu_pool(vp), q.cpu()
    for s in range(2):
        for g in range(hkv):
            Kl = O.logical_rows(kc, table[s], g, n)
            Vl = O.logical_rows(vc, table[s], g, n)
            qg = O.widen(qc[s, g * G:(g + 1) * G])
            ref_g, _ = O.attention(qg, Kl, Vl, O.kept_rows(idx_np[s, g], seg[0], seg[1], n), SCALE)
            ref_d, _ = O.dense_attention(qg, Kl, Vl, SCALE)
            for out in (small, big, det):
                assert_attn(out[0][0, s, g * G:(g + 1) * G], ref_g, f"gather s{s} g{g}")
                assert_attn(out[2][0, s, g * G:(g + 1) * G], ref_d, f"dense s{s} g{g}")
