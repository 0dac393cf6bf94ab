"""Pins of the oracle to facts outside itself.

Each pin is independent of the oracle's own code: a library routine that
computes the same quantity (torch's scaled-dot-product attention and
average pool), hand-derived worked cases (tests/golden/hand_cases.json),
closed forms, invariants that hold for any input, and brute force on tiny
inputs.  A plausible slip in the oracle (a dropped scale, a wrong softmax
axis, an off-by-one causal mask, a reversed tie-break, a transposed
operand) fails at least one of them; test_oracle_mutants.py checks that.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle as O
import synth

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = json.load(open(os.path.join(HERE, "golden", "hand_cases.json")))["cases"]
D = 128
SCALE = 1.0 / math.sqrt(D)


def _q_for_logits(logit_rows):
    """Queries/keys whose scaled dot products equal the given logits:
    q_h = sqrt(d) * e_h and K[i, h] = logit_rows[h][i]."""
    lr = np.asarray(logit_rows, dtype=np.float64)
    G, n = lr.shape
    q = np.zeros((G, D))
    K = np.zeros((n, D))
    for h in range(G):
        q[h, h] = math.sqrt(D)
        K[:, h] = lr[h]
    return q, K


def _rand(rng, *shape):
    """bf16-representable normals as float64."""
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(torch.bfloat16)
    return x.double().numpy()


# --------------------------------------------------------------------------
# golden hand-derived cases
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["softmax_three_keys", "group_sum_two_heads"])
def test_golden_focal_scores(name):
    c = GOLD[name]
    q, K = _q_for_logits(c["logits"])
    s0, s1 = c["segment"]
    got = O.focal_scores(q, K, s0, s1, SCALE, "segment")
    np.testing.assert_allclose(got, c["scores"], rtol=1e-13, atol=0)


def test_golden_context_vs_segment():
    c = GOLD["context_vs_segment"]
    q, K = _q_for_logits(c["logits"])
    s0, s1 = c["segment"]
    np.testing.assert_allclose(O.focal_scores(q, K, s0, s1, SCALE, "segment"), c["scores_segment"], rtol=1e-13)
    np.testing.assert_allclose(O.focal_scores(q, K, s0, s1, SCALE, "context"), c["scores_context"], rtol=1e-13)


def test_golden_topk_ties():
    c = GOLD["topk_ties"]
    for k, want in c["topk"].items():
        assert O.topk(c["scores"], int(k)).tolist() == want


def test_golden_pool():
    c = GOLD["pool_width7"]
    np.testing.assert_allclose(O.avg_pool(c["x"], 7), c["pooled"], rtol=0, atol=1e-15)


def test_golden_attention_two_rows():
    c = GOLD["attention_two_rows"]
    q, K = _q_for_logits(c["logits"])
    V = np.zeros((2, D))
    V[:, :2] = c["v01"]
    out, lse = O.attention(q, K, V, [0, 1], SCALE)
    np.testing.assert_allclose(out[0, :2], c["out01"], rtol=1e-14)
    assert np.all(out[0, 2:] == 0)
    assert abs(lse[0] - c["lse"]) < 1e-14


def test_golden_window_causal_uniform():
    c = GOLD["window_causal_uniform"]
    n, W = c["n"], c["window"]
    qw = np.zeros((W, 1, D))
    K = np.random.default_rng(0).standard_normal((n, D))
    got = O.window_scores(qw, K, 0, n, SCALE, causal=True)
    np.testing.assert_allclose(got, c["scores"], rtol=1e-14)


def test_golden_window_noncausal_uniform():
    c = GOLD["window_noncausal_uniform"]
    n, W = c["n"], c["window"]
    qw = np.zeros((W, 1, D))
    K = np.random.default_rng(0).standard_normal((n, D))
    got = O.window_scores(qw, K, 0, n, SCALE, causal=False)
    np.testing.assert_allclose(got, c["scores"], rtol=1e-14)


def test_golden_window_noncausal_weighted():
    """Window rows with different logits per key: K[i] is the i-th unit
    vector and each row's query holds its logits (scaled by sqrt(d))."""
    c = GOLD["window_noncausal_weighted"]
    lg = np.asarray(c["logits"], dtype=np.float64)
    W, n = lg.shape
    K = np.zeros((n, D))
    K[np.arange(n), np.arange(n)] = 1.0
    qw = np.zeros((W, 1, D))
    qw[:, 0, :n] = lg * math.sqrt(D)
    s0, s1 = c["segment"]
    got = O.window_scores(qw, K, s0, s1, SCALE, causal=False)
    np.testing.assert_allclose(got, c["scores"], rtol=1e-14)


# --------------------------------------------------------------------------
# library routines
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(4))
def test_attention_matches_sdpa(seed):
    rng = np.random.default_rng(seed)
    G, N = int(rng.integers(1, 9)), int(rng.integers(1, 300))
    q, K, V = _rand(rng, G, D), _rand(rng, N, D), _rand(rng, N, D)
    rows = np.sort(rng.choice(N, size=int(rng.integers(1, N + 1)), replace=False))
    out, _ = O.attention(q, K, V, rng.permutation(rows), SCALE)
    tq = torch.from_numpy(q)[None, :, None, :]              # [1, G, 1, d]
    tk = torch.from_numpy(K[rows])[None, None].expand(1, G, -1, -1)
    tv = torch.from_numpy(V[rows])[None, None].expand(1, G, -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[0, :, 0, :].numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("n", [1, 2, 3, 7, 8, 50, 257])
def test_pool_matches_torch(n):
    x = np.random.default_rng(n).random(n)
    ref = torch.nn.functional.avg_pool1d(torch.from_numpy(x)[None, None], 7, 1, 3, count_include_pad=True)[0, 0].numpy()
    np.testing.assert_allclose(O.avg_pool(x, 7), ref, rtol=1e-14, atol=1e-15)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def test_attention_zero_query_is_mean():
    rng = np.random.default_rng(1)
    K, V = _rand(rng, 40, D), _rand(rng, 40, D)
    rows = np.array([3, 9, 17, 33])
    out, lse = O.attention(np.zeros((2, D)), K, V, rows, SCALE)
    np.testing.assert_allclose(out[0], V[rows].mean(0), rtol=1e-13, atol=1e-14)
    assert abs(lse[0] - math.log(4)) < 1e-14


def test_attention_single_row_and_constant_v():
    rng = np.random.default_rng(2)
    q, K, V = _rand(rng, 3, D), _rand(rng, 20, D), _rand(rng, 20, D)
    out, lse = O.attention(q, K, V, [11], SCALE)
    np.testing.assert_array_equal(out, np.repeat(V[11][None], 3, 0))
    np.testing.assert_allclose(lse, (q @ K[11]) * SCALE, rtol=1e-14)
    Vc = np.repeat(V[4][None], 20, 0)
    out, _ = O.attention(q, K, Vc, np.arange(20), SCALE)
    np.testing.assert_allclose(out, np.repeat(V[4][None], 3, 0), rtol=1e-13, atol=1e-14)


def test_window_scores_scale_sensitive():
    """A two-key case where the scale matters: one window row, one head,
    logits 0 and ln 3 after scaling -> weights 1/4, 3/4 (causal row sees both)."""
    q = np.zeros((1, 1, D))
    q[0, 0, 0] = math.sqrt(D)
    K = np.zeros((2, D))
    K[1, 0] = math.log(3)
    np.testing.assert_allclose(O.window_scores(q, K, 0, 2, SCALE), [0.25, 0.75], rtol=1e-13)


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

@pytest.mark.parametrize("G", [1, 2, 4])
def test_score_sums(G):
    rng = np.random.default_rng(G)
    N, s0, s1 = 300, 20, 250
    q, K = _rand(rng, G, D), _rand(rng, N, D)
    seg = O.focal_scores(q, K, s0, s1, SCALE, "segment")
    assert abs(seg.sum() - G) < 1e-12 and seg.shape == (s1 - s0,)
    ctx_in = O.focal_scores(q, K, s0, s1, SCALE, "context")
    ctx_all = O.focal_scores(q, K, 0, N, SCALE, "context")
    assert abs(ctx_all.sum() - G) < 1e-12
    np.testing.assert_allclose(ctx_all[s0:s1], ctx_in, rtol=1e-14)
    assert np.all(ctx_in < seg)
    W = 8
    qw = _rand(rng, W, G, D)
    ws = O.window_scores(qw, K, 0, N, SCALE, causal=True)
    assert abs(ws.sum() - W * G) < 1e-11
    # the causal window: key N-1 is seen only by the last window row
    qw2 = qw.copy()
    qw2[:-1] *= 0.0
    ws2 = O.window_scores(qw2, K, 0, N, SCALE, causal=True)
    assert abs(ws2.sum() - W * G) < 1e-11


def test_score_permutation_equivariance():
    rng = np.random.default_rng(5)
    N = 120
    q, K = _rand(rng, 2, D), _rand(rng, N, D)
    perm = rng.permutation(N)
    a = O.focal_scores(q, K, 0, N, SCALE, "segment")
    b = O.focal_scores(q, K[perm], 0, N, SCALE, "segment")
    np.testing.assert_allclose(b, a[perm], rtol=1e-13)


def _brute_topk(s, k):
    """The unique k-subset S with: for i in S, j not in S, s_i > s_j or
    (s_i == s_j and i < j).  Enumerates every subset."""
    n = len(s)
    found = []
    for S in itertools.combinations(range(n), k):
        Sset = set(S)
        ok = all((s[i] > s[j]) or (s[i] == s[j] and i < j)
                 for i in S for j in range(n) if j not in Sset)
        if ok:
            found.append(list(S))
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 11))
    # few distinct values so that ties are common
    s = rng.integers(0, 4, size=n).astype(np.float32) / 4
    for k in range(1, n + 1):
        assert O.topk(s, k).tolist() == _brute_topk(s.tolist(), k)


def test_topk_all_equal_and_budget_count():
    s = np.full(3584, 1.0 / 3584, dtype=np.float32)
    assert O.topk(s, 179).tolist() == list(range(179))
    rng = np.random.default_rng(9)
    for cfg in (synth.C0, synth.C1, synth.C4):
        sc = rng.random(cfg.n_visual)
        keep = O.topk(sc, cfg.k)
        assert keep.shape[0] == cfg.k and len(np.unique(keep)) == cfg.k
        n = cfg.prefix_len + 5
        R = O.kept_rows(keep, 0, cfg.n_visual, n)
        assert len(np.unique(R)) == cfg.k + (n - cfg.n_visual)
    assert (synth.C0.k, synth.C1.k, synth.C2.k, synth.C4.k, synth.C3.k) == (179, 320, 6554, 154, 2048)


@pytest.mark.parametrize("seed", range(5))
def test_topk_warm_equals_cold(seed):
    rng = np.random.default_rng(seed)
    n, k = 500, 25
    s = (rng.integers(0, 40, size=n) / 40).astype(np.float32)
    cold = O.topk(s, k)
    for _ in range(10):
        warm = np.sort(rng.choice(n, size=k, replace=False))
        assert O.topk_warm(s, k, warm).tolist() == cold.tolist()
    assert O.topk_warm(s, k, cold).tolist() == cold.tolist()


def test_full_budget_is_dense():
    rng = np.random.default_rng(3)
    N, s0, s1 = 200, 10, 150
    q, K, V = _rand(rng, 2, D), _rand(rng, N, D), _rand(rng, N, D)
    sc = O.focal_scores(q, K, s0, s1, SCALE)
    keep = O.topk(sc, s1 - s0)
    out_s, lse_s = O.attention(q, K, V, O.kept_rows(keep, s0, s1, N), SCALE)
    out_d, lse_d = O.dense_attention(q, K, V, SCALE)
    np.testing.assert_array_equal(out_s, out_d)
    np.testing.assert_array_equal(lse_s, lse_d)


def test_tie_band_check():
    rng = np.random.default_rng(4)
    sc = rng.random(100)
    k = 10
    o = O.topk(sc, k)
    assert O.tie_band_check(o, sc, k) == (True, 0)
    sc2 = sc.copy()
    order = np.argsort(-sc2)
    sc2[order[k]] = sc2[order[k - 1]] * (1 - 1e-7)     # a near tie at the boundary
    o2 = O.topk(sc2, k)
    swapped = np.sort(np.concatenate([np.setdiff1d(o2, [order[k - 1]]), [order[k]]]))
    assert O.tie_band_check(swapped, sc2, k)[0]
    far = np.sort(np.concatenate([o[1:], [order[-1]]]))
    assert not O.tie_band_check(far, sc, k)[0]
    assert not O.tie_band_check(o[:-1], sc, k)[0]
    assert not O.tie_band_check(np.concatenate([o[:-1], o[:1]]), sc, k)[0]


# --------------------------------------------------------------------------
# KV store and schedule
# --------------------------------------------------------------------------

def test_logical_rows_inverts_scatter():
    rng = np.random.default_rng(7)
    blk, hkv, n = 16, 3, 100
    rows = _rand(rng, hkv, n, 8)
    nb = -(-n // blk)
    phys = rng.permutation(nb + 4)[:nb]
    pool = np.zeros((nb + 4, hkv, blk, 8))
    for j in range(n):
        pool[phys[j // blk], :, j % blk, :] = rows[:, j, :]
    for g in range(hkv):
        np.testing.assert_array_equal(O.logical_rows(pool, phys, g, n, blk), rows[g])


def test_shared_prefix_table_reads_same_prefix():
    from synth.gen import shared_prefix_table
    table, nb = shared_prefix_table(4, np.array([2, 5, 1]))
    rng = np.random.default_rng(8)
    pool = rng.standard_normal((nb, 2, 16, 8))
    a = O.logical_rows(pool, table[0], 1, 64)
    b = O.logical_rows(pool, table[2], 1, 64)
    np.testing.assert_array_equal(a, b)
    c = O.logical_rows(pool, table[1], 1, 64 + 80)
    assert not np.array_equal(c[64:80], O.logical_rows(pool, table[0], 1, 80)[64:80])


def test_layer_plan_c1():
    p0 = O.focal_layer_plan(28, (3, 14), 0)
    assert [e[0] for e in p0[:3]] == ["dense"] * 3
    assert p0[3] == ("focal", 3) and p0[14] == ("focal", 14)
    assert all(p0[l] == ("sparse", l, 0, 3) for l in range(4, 14))
    assert all(p0[l] == ("sparse", l, 0, 14) for l in range(15, 28))
    p5 = O.focal_layer_plan(28, (3, 14), 5)
    assert all(p5[l] == ("sparse", l, 4, 14) for l in range(3))


def test_gather_rows_exact():
    src = np.arange(40 * 6).reshape(40, 6)
    got = O.gather_rows(src, [3, 7, 20], 36, 4)
    np.testing.assert_array_equal(got, src[[3, 7, 20, 36, 37, 38, 39]])


# --------------------------------------------------------------------------
# focal-layer profiling (FastOCR, Focal-Guided Pruning, "Focal Layer
# Selection"): the image-attention ratio and the choice of the focal layers
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(4))
def test_visual_mass_matches_sdpa_indicator(seed):
    """The ratio is attention whose value rows are the segment's indicator:
    torch's scaled_dot_product_attention (fp64, CPU) with V[i] = [i in seg]."""
    rng = np.random.default_rng(100 + seed)
    G, N = int(rng.integers(1, 9)), int(rng.integers(2, 400))
    s0 = int(rng.integers(0, N))
    s1 = int(rng.integers(s0, N + 1))
    q, K = _rand(rng, G, D) * 3.0, _rand(rng, N, D)
    ind = np.zeros((N, 1))
    ind[s0:s1] = 1.0
    tq = torch.from_numpy(q)[None, :, None, :]
    tk = torch.from_numpy(K)[None, None].expand(1, G, -1, -1)
    tv = torch.from_numpy(ind)[None, None].expand(1, G, -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=SCALE)[0, :, 0, 0].numpy()
    np.testing.assert_allclose(O.visual_mass(q, K, s0, s1, SCALE), ref, rtol=1e-12, atol=1e-14)


def test_visual_mass_closed_forms():
    rng = np.random.default_rng(7)
    N, G = 300, 4
    K = _rand(rng, N, D)
    # a zero query attends uniformly: the ratio is the segment's share of rows
    np.testing.assert_allclose(O.visual_mass(np.zeros((G, D)), K, 40, 250, SCALE), np.full(G, 210 / 300), rtol=1e-14)
    q = _rand(rng, G, D)
    np.testing.assert_allclose(O.visual_mass(q, K, 0, N, SCALE), np.ones(G), rtol=1e-14)   # everything
    np.testing.assert_allclose(O.visual_mass(q, K, 77, 77, SCALE), np.zeros(G), atol=0)   # empty segment
    # a query aligned with one segment key puts (almost) all its mass there
    q1 = np.tile(K[120] * 60.0, (G, 1))
    assert np.all(O.visual_mass(q1, K, 100, 130, SCALE) > 0.999)
    assert np.all(O.visual_mass(q1, K, 0, 100, SCALE) < 1e-3)


def test_pick_focal_layers_cases():
    # dyadic ratios, so equal means are equal exactly: means .25 .5 .25 .5 .5
    r = np.array([[0.125, 0.375], [0.5, 0.5], [0.25, 0.25], [0.875, 0.125], [0.5, 0.5]])
    # three layers tie at 0.5: the lower indices win
    assert list(O.pick_focal_layers(r, 2)) == [1, 3]
    assert list(O.pick_focal_layers(r, 3)) == [1, 3, 4]
    assert list(O.pick_focal_layers(r, 4)) == [0, 1, 3, 4]
    assert list(O.pick_focal_layers(r, 5)) == [0, 1, 2, 3, 4]
    # the mean, not the peak, decides
    r2 = np.array([[0.0, 0.0, 1.0], [0.4, 0.4, 0.4]])
    assert list(O.pick_focal_layers(r2, 1)) == [1]


def test_pick_focal_layers_exact_means():
    """Means that fp64 summation would round together are told apart, and
    means that are equal only as exact sums tie (to the lower layer), in
    whatever order the terms come.  Layer 0: 2^-60 + 2^-60 + 1 (a left-to-right
    fp64 sum rounds it to 1); layer 1: exactly 1; layer 2: 1 + 2^-59 + 0, the
    same exact sum as layer 0; layer 3: the terms of layer 0 reversed."""
    t = 2.0 ** -60
    r = np.array([[t, t, 1.0], [1.0, 0.0, 0.0], [1.0, 2 * t, 0.0], [1.0, t, t]])
    assert list(O.pick_focal_layers(r, 1)) == [0]
    assert list(O.pick_focal_layers(r, 3)) == [0, 2, 3]
    assert list(O.pick_focal_layers(r[[1, 0]], 1)) == [1]        # layer 1 of this pair holds the larger sum
    assert list(O.pick_focal_layers(np.array([[np.nan, 0.5], [0.5, 0.0]]), 1)) == [0]   # NaN counts as 0: a tie


@pytest.mark.parametrize("seed", range(3))
def test_pick_focal_layers_brute_force(seed):
    """Every n_pick-subset of layers: the chosen one has the largest sum of
    means, and among equal sums the lexicographically smallest layers."""
    rng = np.random.default_rng(seed)
    L = 6
    r = rng.integers(0, 4, size=(L, 3)) / 4.0   # many ties
    mean = r.mean(axis=1)
    for n_pick in range(1, L + 1):
        best = None
        for sub in itertools.combinations(range(L), n_pick):
            # rank order: a subset is better if its sorted means are larger
            key = sorted(((-mean[l], l) for l in sub))
            if best is None or key < best[0]:
                best = (key, sub)
        assert list(O.pick_focal_layers(r, n_pick)) == list(best[1])


# --------------------------------------------------------------------------
# fork lifecycle (HPD-Parsing wiki, inference scheduling: fork pointer, zero
# copy, reference-counted release)
# --------------------------------------------------------------------------

def _scatter(rng, pool, table, rows, start=0):
    for j in range(rows.shape[1]):
        pos = start + j
        pool[table[pos // 16], :, pos % 16, :] = rows[:, j, :]


@pytest.mark.parametrize("L", [0, 5, 16, 37, 64, 79])
def test_fork_child_sees_parent_rows_and_stays_isolated(L):
    rng = np.random.default_rng(L)
    hkv, d, nb = 2, 8, 20
    pool = np.zeros((nb, hkv, 16, d))
    parent = np.full(8, -1)
    parent[:6] = [3, 11, 4, 17, 8, 0]
    _scatter(rng, pool, parent, rng.standard_normal((hkv, L, d)))
    child = O.fork_child_table(parent, L, new_block=19)
    pool2 = O.copy_block(pool, parent[L // 16], 19) if L % 16 else pool
    for g in range(hkv):   # the child reads the parent's rows before the fork, bit for bit
        np.testing.assert_array_equal(O.logical_rows(pool2, child, g, L), O.logical_rows(pool, parent, g, L))
    # blocks wholly before the fork are shared; a partly filled one is a fresh copy
    assert list(child[:L // 16]) == list(parent[:L // 16])
    assert (L % 16 == 0) == (19 not in child)
    # both append 9 rows after the fork point: neither sees the other's
    if L + 9 <= 6 * 16 and L % 16:
        before_c = O.logical_rows(pool2, child, 0, L)
        before_p = O.logical_rows(pool2, parent, 0, L)
        pnew, cnew = rng.standard_normal((hkv, 9, d)), rng.standard_normal((hkv, 9, d))
        child_ext = child.copy()   # fresh blocks for the child's rows past its copied block
        for i, blk in zip(range(L // 16 + 1, (L + 8) // 16 + 1), [1, 2, 5, 6, 7]):
            child_ext[i] = blk
        _scatter(rng, pool2, parent, pnew, start=L)
        _scatter(rng, pool2, child_ext, cnew, start=L)
        np.testing.assert_array_equal(O.logical_rows(pool2, child_ext, 0, L), before_c)
        np.testing.assert_array_equal(O.logical_rows(pool2, parent, 0, L), before_p)
        np.testing.assert_array_equal(O.logical_rows(pool2, parent, 0, L + 9)[L:], pnew[0])
        np.testing.assert_array_equal(O.logical_rows(pool2, child_ext, 0, L + 9)[L:], cnew[0])


# --------------------------------------------------------------------------
# draft verification (HPD-Parsing wiki, P-MTP: drafts verified in parallel)
# --------------------------------------------------------------------------

def test_verify_attention_matches_causal_sdpa():
    """Over every row, m drafts at the end of the sequence: torch's causal
    scaled_dot_product_attention on the last m query positions (fp64)."""
    rng = np.random.default_rng(21)
    n, m, G = 90, 6, 2
    K, V = _rand(rng, n, D), _rand(rng, n, D)
    qd = _rand(rng, m, G, D)
    out, _ = O.verify_attention(qd, K, V, np.arange(n), n, SCALE)
    # causal SDPA over the full sequence, with the drafts' queries in the last m positions
    Q = np.zeros((G, n, D))
    Q[:, n - m:, :] = qd.transpose(1, 0, 2)
    tq = torch.from_numpy(Q)[None]
    tk = torch.from_numpy(K)[None, None].expand(1, G, -1, -1)
    tv = torch.from_numpy(V)[None, None].expand(1, G, -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=SCALE)[0].numpy()
    np.testing.assert_allclose(out, ref[:, n - m:, :].transpose(1, 0, 2), rtol=1e-12, atol=1e-12)


def test_verify_attention_single_draft_is_attention():
    rng = np.random.default_rng(22)
    n = 50
    K, V = _rand(rng, n, D), _rand(rng, n, D)
    rows = np.sort(rng.choice(n - 1, size=20, replace=False).tolist() + [n - 1])
    qd = _rand(rng, 1, 4, D)
    out, lse = O.verify_attention(qd, K, V, rows, n, SCALE)
    ref, rl = O.attention(qd[0], K, V, rows, SCALE)
    np.testing.assert_array_equal(out[0], ref)
    # the first of two drafts does not see the second
    out2, _ = O.verify_attention(_rand(rng, 2, 4, D) * 0 + qd, K, V, rows, n, SCALE)
    ref1, _ = O.attention(qd[0], K, V, [x for x in rows if x <= n - 2], SCALE)
    np.testing.assert_allclose(out2[0], ref1, rtol=1e-14)


# --------------------------------------------------------------------------
# TSP stage 2 (FastKV 2A: later layers run over the propagated tokens only)
# --------------------------------------------------------------------------

def test_causal_prefill_matches_causal_sdpa():
    """Every (position, head): torch's causal scaled_dot_product_attention in
    fp64 with each kv head repeated over its G query heads."""
    rng = np.random.default_rng(31)
    n, hkv, G = 37, 3, 2
    Q = _rand(rng, n, hkv * G, D)
    K, V = _rand(rng, n, hkv, D), _rand(rng, n, hkv, D)
    out, lse = O.causal_prefill(Q, K, V, SCALE)
    tq = torch.from_numpy(Q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
    tv = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=SCALE)[0]
    ref = ref.permute(1, 0, 2).reshape(n * hkv * G, D).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    # lse: the log of the causal normaliser, written out for a few rows
    S = np.einsum("ihd,jhd->hij", Q, np.repeat(K, G, axis=1)) * SCALE
    for i, h in [(0, 0), (5, 3), (n - 1, hkv * G - 1)]:
        assert abs(lse[i * hkv * G + h] - np.log(np.exp(S[h, i, : i + 1]).sum())) < 1e-12


def test_causal_prefill_ends():
    """The first token sees only itself (out = its V row); the last sees the
    whole sequence (dense attention); a sampled row equals the full run."""
    rng = np.random.default_rng(32)
    n, hkv, G = 20, 2, 4
    Q = _rand(rng, n, hkv * G, D)
    K, V = _rand(rng, n, hkv, D), _rand(rng, n, hkv, D)
    out, lse = O.causal_prefill(Q, K, V, SCALE, rows=[(0, h) for h in range(hkv * G)])
    for h in range(hkv * G):
        np.testing.assert_array_equal(out[h], V[0, h // G])
        assert abs(lse[h] - SCALE * float(Q[0, h] @ K[0, h // G])) < 1e-12
    last, _ = O.causal_prefill(Q, K, V, SCALE, rows=[(n - 1, 5)])
    np.testing.assert_allclose(last[0], O.dense_attention(Q[n - 1, 5][None], K[:, 1], V[:, 1], SCALE)[0][0],
                               rtol=1e-14)
    full, _ = O.causal_prefill(Q, K, V, SCALE)
    one, _ = O.causal_prefill(Q, K, V, SCALE, rows=[(13, 6)])
    np.testing.assert_array_equal(one[0], full[13 * hkv * G + 6])


# --------------------------------------------------------------------------
# merging two partial attentions (shared rows apart from a branch's own rows)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [41, 42])
def test_merge_attention_equals_union(seed):
    """Attention over A and over B, merged, equals attention over A u B
    (A, B disjoint); either part empty leaves the other unchanged."""
    rng = np.random.default_rng(seed)
    n, G = 80, 3
    K, V = _rand(rng, n, D), _rand(rng, n, D)
    qg = _rand(rng, G, D)
    perm = rng.permutation(n)
    A, B = np.sort(perm[:30]), np.sort(perm[30:])
    oa, la = O.attention(qg, K, V, A, SCALE)
    ob, lb = O.attention(qg, K, V, B, SCALE)
    ou, lu = O.attention(qg, K, V, np.arange(n), SCALE)
    om, lm = O.merge_attention(oa, la, ob, lb)
    np.testing.assert_allclose(om, ou, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lm, lu, rtol=1e-13)
    om2, _ = O.merge_attention(ob, lb, oa, la)
    np.testing.assert_allclose(om2, ou, rtol=1e-12, atol=1e-13)
    empty_o, empty_l = np.zeros_like(oa), np.full(G, -np.inf)
    oe, le = O.merge_attention(oa, la, empty_o, empty_l)
    np.testing.assert_array_equal(oe, oa)
    np.testing.assert_array_equal(le, la)
    oz, lz = O.merge_attention(empty_o, empty_l, empty_o, empty_l)
    assert np.all(oz == 0) and np.all(np.isneginf(lz))


# --------------------------------------------------------------------------
# many instances per call (the full-size parity checks use these forms)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(3))
def test_attention_masked_matches_sdpa(seed):
    """Masked attention against torch's scaled-dot-product attention with a
    boolean mask, several (batch, query) instances at once; a query whose
    mask is empty gets out = 0 and lse = -inf."""
    rng = np.random.default_rng(100 + seed)
    B, Q, N = 3, int(rng.integers(1, 9)), int(rng.integers(1, 200))
    q, K, V = _rand(rng, B, Q, D), _rand(rng, B, N, D), _rand(rng, B, N, D)
    vis = rng.random((B, Q, N)) < 0.3
    vis[:, 0, :] = True
    vis[1, -1, :] = False                            # nothing visible
    out, lse = O.attention_masked(q, K, V, vis, SCALE)
    ok = vis.any(axis=-1)
    tq, tk, tv = (torch.from_numpy(x)[:, None] for x in (q, K, V))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(vis)[:, None])[:, 0]
    np.testing.assert_allclose(out[ok], ref.numpy()[ok], rtol=1e-12, atol=1e-12)
    assert np.all(out[~ok] == 0) and np.all(np.isneginf(lse[~ok]))
    s = (q @ np.swapaxes(K, 1, 2)) * SCALE
    ref_lse = np.log(np.where(vis, np.exp(s), 0.0).sum(-1)[ok])
    np.testing.assert_allclose(lse[ok], ref_lse, rtol=1e-12)


def test_attention_masked_equals_attention_over_rows():
    """Each masked instance equals attention over the rows its mask selects."""
    rng = np.random.default_rng(7)
    q, K, V = _rand(rng, 4, 2, D), _rand(rng, 4, 300, D), _rand(rng, 4, 300, D)
    vis = rng.random((4, 1, 300)) < 0.1
    out, lse = O.attention_masked(q, K, V, vis, SCALE)
    for b in range(4):
        ref, rl = O.attention(q[b], K[b], V[b], np.nonzero(vis[b, 0])[0], SCALE)
        np.testing.assert_allclose(out[b], ref, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[b], rl, rtol=1e-13)


def test_batched_scores_topk_and_tie_band_equal_per_row():
    """Focal scores, top-k and the tie-band rule over rows equal one call
    per row (which the pins above fix)."""
    rng = np.random.default_rng(8)
    q, K = _rand(rng, 5, 2, D), _rand(rng, 5, 90, D)
    sc = O.focal_scores(q, K, 10, 80, SCALE)
    for b in range(5):
        np.testing.assert_array_equal(sc[b], O.focal_scores(q[b], K[b], 10, 80, SCALE))
    k = 7
    idx = O.topk(sc, k)
    for b in range(5):
        np.testing.assert_array_equal(idx[b], O.topk(sc[b], k))
    bad = idx.copy()
    bad[2, 0] = np.argsort(sc[2])[0] if np.argsort(sc[2])[0] not in idx[2] else np.argsort(sc[2])[1]
    bad[2] = np.sort(bad[2])
    bad[3, 1] = bad[3, 0]                            # a repeated index
    ok, nd = O.tie_band_check(bad, sc, k)
    for b in range(5):
        assert (bool(ok[b]), int(nd[b])) == O.tie_band_check(bad[b], sc[b], k)
    assert list(ok) == [True, True, False, False, True]


@pytest.mark.parametrize("n", [1, 7, 50])
def test_pool_rows_match_torch(n):
    x = np.random.default_rng(n).random((3, n))
    ref = torch.nn.functional.avg_pool1d(torch.from_numpy(x)[:, None], 7, 1, 3, count_include_pad=True)[:, 0].numpy()
    np.testing.assert_allclose(O.avg_pool(x, 7), ref, rtol=1e-14, atol=1e-15)
