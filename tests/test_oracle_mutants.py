"""The pins catch plausible mistakes.

Each case plants one slip in the oracle (on the CPU, by swapping one of its
functions for a wrong variant) and checks that at least one pin from
test_oracle_pins.py then fails.
"""
import numpy as np
import pytest

from oracle import oracle as O
from tests import test_oracle_pins as P

F64 = np.float64


def _no_scale(q, K, scale):
    return np.asarray(q, F64) @ np.asarray(K, F64).T


def _softmax_axis0(s):
    s = np.asarray(s, F64)
    m = s.max(axis=0, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=0, keepdims=True)


def _topk_high_index_wins(scores, k):
    s32 = np.asarray(scores, dtype=np.float32).astype(F64)
    n = s32.shape[0]
    order = np.lexsort((-np.arange(n), -s32))
    return np.sort(order[:k])


def _window_off_by_one(qw, K, s0, s1, scale, causal=True):
    qw = np.asarray(qw, F64)
    K = np.asarray(K, F64)
    N, W = K.shape[0], qw.shape[0]
    acc = np.zeros(N)
    for r in range(W):
        vis = max(N - W + r, 1)
        acc[:vis] += O.softmax(O.logits(qw[r], K[:vis], scale)).sum(0)
    return acc[s0:s1]


def _window_always_causal(qw, K, s0, s1, scale, causal=True):
    return _window_reference(qw, K, s0, s1, scale, lambda pos, N: pos + 1)


def _window_noncausal_misses_last_key(qw, K, s0, s1, scale, causal=True):
    return _window_reference(qw, K, s0, s1, scale, lambda pos, N: pos + 1 if causal else N - 1)


def _window_reference(qw, K, s0, s1, scale, visible):
    qw = np.asarray(qw, F64)
    K = np.asarray(K, F64)
    N, W = K.shape[0], qw.shape[0]
    acc = np.zeros(N)
    for r in range(W):
        vis = visible(N - W + r, N)
        acc[:vis] += O.softmax(O.logits(qw[r], K[:vis], scale)).sum(0)
    return acc[s0:s1]


def _attention_uses_k_for_v(qg, K, V, rows, scale):
    r = np.unique(np.asarray(rows, dtype=np.int64))
    s = O.logits(qg, np.asarray(K, F64)[r], scale)
    m = s.max(1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(1, keepdims=True)
    return (e @ np.asarray(K, F64)[r]) / z, (m + np.log(z))[:, 0]


def _pool_excluding_pad(x, width):
    x = np.asarray(x, F64)
    h = width // 2
    out = np.empty_like(x)
    for i in range(len(x)):
        lo, hi = max(0, i - h), min(len(x), i + h + 1)
        out[i] = x[lo:hi].mean()
    return out


def _kept_rows_unshifted(idx, s0, s1, n):
    idx = np.asarray(idx, dtype=np.int64)
    return np.concatenate([idx, np.arange(0, s0), np.arange(s1, n)])


def _focal_sum_over_keys(qg, K, s0, s1, scale, norm="segment"):
    s = O.logits(qg, K, scale)
    p = O.softmax(s[:, s0:s1])
    return p.sum(axis=1).repeat(s1 - s0)[: s1 - s0]


def _warm_uses_max(scores, k, warm):
    s32 = np.asarray(scores, dtype=np.float32)
    theta = s32[np.asarray(warm)].max()
    cand = np.nonzero(s32 >= theta)[0]
    if cand.shape[0] < k:
        return cand
    return cand[O.topk(s32[cand], k)]


def _mass_segment_softmax(qg, K, s0, s1, scale):
    if s1 <= s0:
        return np.zeros(np.asarray(qg).shape[0])
    return O.softmax(O.logits(qg, np.asarray(K, F64)[s0:s1], scale)).sum(axis=1)


def _pick_high_layer_wins(ratios, n_pick):
    r = np.asarray(ratios, F64)
    mean = r.mean(axis=1)
    order = np.lexsort((-np.arange(r.shape[0]), -mean))
    return np.sort(order[:n_pick])


def _pick_by_peak(ratios, n_pick):
    r = np.asarray(ratios, F64)
    order = np.lexsort((np.arange(r.shape[0]), -r.max(axis=1)))
    return np.sort(order[:n_pick])


def _masked_ignores_mask(q, K, V, visible, scale):
    s = O.logits(q, K, scale)
    e = np.exp(s - s.max(-1, keepdims=True))
    z = e.sum(-1, keepdims=True)
    return (e @ np.asarray(V, F64)) / z, (s.max(-1, keepdims=True) + np.log(z))[..., 0]


def _masked_shifted_mask(q, K, V, visible, scale):
    vis = np.roll(np.broadcast_to(np.asarray(visible, bool), O.logits(q, K, scale).shape), 1, axis=-1)
    return _masked_reference(q, K, V, vis, scale)


def _masked_reference(q, K, V, visible, scale):
    s = np.where(visible, O.logits(q, K, scale), -np.inf)
    m = s.max(-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m)
    z = e.sum(-1, keepdims=True)
    return (e @ np.asarray(V, F64)) / np.where(z > 0, z, 1.0), (m + np.log(np.where(z > 0, z, 1.0)))[..., 0]


MUTANTS = [
    ("logits", _no_scale, [P.test_attention_matches_sdpa, P.test_window_scores_scale_sensitive]),
    ("softmax", _softmax_axis0, [lambda: P.test_score_sums(2), lambda: P.test_golden_focal_scores("softmax_three_keys")]),
    ("topk", _topk_high_index_wins, [lambda: P.test_topk_brute_force(0), P.test_golden_topk_ties]),
    ("window_scores", _window_off_by_one, [P.test_golden_window_causal_uniform]),
    ("window_scores", _window_always_causal, [P.test_golden_window_noncausal_uniform,
                                              P.test_golden_window_noncausal_weighted]),
    ("window_scores", _window_noncausal_misses_last_key, [P.test_golden_window_noncausal_uniform,
                                                          P.test_golden_window_noncausal_weighted]),
    ("attention", _attention_uses_k_for_v, [lambda: P.test_attention_matches_sdpa(0)]),
    ("avg_pool", _pool_excluding_pad, [lambda: P.test_pool_matches_torch(8), P.test_golden_pool]),
    ("kept_rows", _kept_rows_unshifted, [P.test_full_budget_is_dense]),
    ("focal_scores", _focal_sum_over_keys, [lambda: P.test_golden_focal_scores("group_sum_two_heads")]),
    ("topk_warm", _warm_uses_max, [lambda: P.test_topk_warm_equals_cold(0)]),
    ("visual_mass", _mass_segment_softmax, [P.test_visual_mass_closed_forms, lambda: P.test_visual_mass_matches_sdpa_indicator(0)]),
    ("pick_focal_layers", _pick_high_layer_wins, [P.test_pick_focal_layers_cases, lambda: P.test_pick_focal_layers_brute_force(0)]),
    ("pick_focal_layers", _pick_by_peak, [P.test_pick_focal_layers_cases]),
    ("attention_masked", _masked_ignores_mask, [lambda: P.test_attention_masked_matches_sdpa(0),
                                                P.test_attention_masked_equals_attention_over_rows]),
    ("attention_masked", _masked_shifted_mask, [lambda: P.test_attention_masked_matches_sdpa(0),
                                                P.test_attention_masked_equals_attention_over_rows]),
]


@pytest.mark.parametrize("name,bad,pins", MUTANTS, ids=[f"{m[0]}-{m[1].__name__}" for m in MUTANTS])
def test_pins_catch_mutant(monkeypatch, name, bad, pins):
    monkeypatch.setattr(O, name, bad)
    for pin in pins:
        fn = pin
        if getattr(pin, "__code__", None) is not None and pin.__code__.co_argcount == 1:
            fn = lambda p=pin: p(0)    # noqa: E731  seeded pins take a seed
        with pytest.raises((AssertionError, ValueError, IndexError)):
            fn()


def _fork_shares_partial(parent_table, parent_len, new_block, block=16):
    t = np.full(np.asarray(parent_table).shape, -1, dtype=np.int64)
    n = -(-parent_len // block)
    t[:n] = np.asarray(parent_table)[:n]
    return t


def test_fork_pin_catches_shared_partial_block(monkeypatch):
    monkeypatch.setattr(O, "fork_child_table", _fork_shares_partial)
    with pytest.raises(AssertionError):
        P.test_fork_child_sees_parent_rows_and_stays_isolated(37)


def _verify_not_causal(qd, K, V, rows, n, scale):
    qd = np.asarray(qd, F64)
    outs, lses = zip(*[O.attention(qd[r], K, V, np.unique(rows), scale) for r in range(qd.shape[0])])
    return np.stack(outs), np.stack(lses)


def _verify_off_by_one(qd, K, V, rows, n, scale):
    qd = np.asarray(qd, F64)
    r_all = np.unique(np.asarray(rows))
    outs, lses = zip(*[O.attention(qd[r], K, V, r_all[r_all < max(n - qd.shape[0] + r, 1)], scale)
                       for r in range(qd.shape[0])])
    return np.stack(outs), np.stack(lses)


@pytest.mark.parametrize("bad", [_verify_not_causal, _verify_off_by_one])
def test_verify_pin_catches(monkeypatch, bad):
    monkeypatch.setattr(O, "verify_attention", bad)
    with pytest.raises(AssertionError):
        P.test_verify_attention_matches_causal_sdpa()


def _prefill_sees_one_less(Q, K, V, scale, rows=None):
    Q, K, V = np.asarray(Q, F64), np.asarray(K, F64), np.asarray(V, F64)
    G = Q.shape[1] // K.shape[1]
    rows = rows or [(i, h) for i in range(Q.shape[0]) for h in range(Q.shape[1])]
    res = [O.attention(Q[i, h][None], K[:, h // G], V[:, h // G], np.arange(max(i, 1)), scale) for i, h in rows]
    return np.stack([o[0] for o, _ in res]), np.array([l[0] for _, l in res])


def _prefill_head_modulo(Q, K, V, scale, rows=None):
    Q, K, V = np.asarray(Q, F64), np.asarray(K, F64), np.asarray(V, F64)
    hkv = K.shape[1]
    rows = rows or [(i, h) for i in range(Q.shape[0]) for h in range(Q.shape[1])]
    res = [O.attention(Q[i, h][None], K[:, h % hkv], V[:, h % hkv], np.arange(i + 1), scale) for i, h in rows]
    return np.stack([o[0] for o, _ in res]), np.array([l[0] for _, l in res])


def _prefill_not_causal(Q, K, V, scale, rows=None):
    Q, K, V = np.asarray(Q, F64), np.asarray(K, F64), np.asarray(V, F64)
    n, G = Q.shape[0], Q.shape[1] // K.shape[1]
    rows = rows or [(i, h) for i in range(n) for h in range(Q.shape[1])]
    res = [O.attention(Q[i, h][None], K[:, h // G], V[:, h // G], np.arange(n), scale) for i, h in rows]
    return np.stack([o[0] for o, _ in res]), np.array([l[0] for _, l in res])


@pytest.mark.parametrize("bad", [_prefill_sees_one_less, _prefill_head_modulo, _prefill_not_causal])
@pytest.mark.parametrize("pin", ["test_causal_prefill_matches_causal_sdpa", "test_causal_prefill_ends"])
def test_prefill_pins_catch(monkeypatch, bad, pin):
    monkeypatch.setattr(O, "causal_prefill", bad)
    with pytest.raises(AssertionError):
        getattr(P, pin)()


def _merge_unweighted(o1, lse1, o2, lse2):
    out = (np.asarray(o1, F64) + np.asarray(o2, F64)) / 2
    return out, np.logaddexp(lse1, lse2)


def _merge_swapped_weights(o1, lse1, o2, lse2):
    l1, l2 = np.asarray(lse1, F64), np.asarray(lse2, F64)
    m = np.maximum(l1, l2)
    w1, w2 = np.exp(l1 - m), np.exp(l2 - m)
    return (np.asarray(o1, F64) * w2[..., None] + np.asarray(o2, F64) * w1[..., None]) / (w1 + w2)[..., None], \
        m + np.log(w1 + w2)


@pytest.mark.parametrize("bad", [_merge_unweighted, _merge_swapped_weights])
def test_merge_pin_catches(monkeypatch, bad):
    monkeypatch.setattr(O, "merge_attention", bad)
    with pytest.raises(AssertionError):
        P.test_merge_attention_equals_union(41)


def test_merge_pin_catches_wrong_lse(monkeypatch):
    real = O.merge_attention

    def bad(o1, lse1, o2, lse2):
        out, _ = real(o1, lse1, o2, lse2)
        return out, np.maximum(np.asarray(lse1, F64), np.asarray(lse2, F64))
    monkeypatch.setattr(O, "merge_attention", bad)
    with pytest.raises(AssertionError):
        P.test_merge_attention_equals_union(41)
