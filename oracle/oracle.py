"""Oracle for the score -> head-sum -> top-k -> sparse-attention path.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow, CPU definition
that the HIP path is checked against.  Only the test suite, the smoke
check and the CPU-baseline leg of the benchmark may import it; the product
path never calls it.  It shares no code with the HIP library.

Precision: inputs are bf16, widened exactly to float64; every dot product,
softmax and attention sum is evaluated in float64.  The one integer
decision (which k tokens to keep) is taken on the scores rounded to
float32, the precision the kernels decide in, with ties to the lower index.

Shapes: the scoring, selection and attention functions take leading batch
dimensions (several sequences, heads or steps at once) and apply the same
definition to each; one call on a single group is the plain case.

Sources (the pages' titles and sections; no formula for the score is
printed there, the readings below are the plainest ones the text supports):

* FastOCR: Dynamic Visual Fixation via KV Cache Pruning (technical summary,
  Methodology / Focal-Guided Pruning, "Cross-Layer Propagation"): focal
  layers attend over the full KV cache, pick the top-attended image tokens
  at kept ratio tau, and every other layer attends only to that set.
* same page, "Cross-Step Fixation Reuse": a non-focal first layer inherits
  the deepest focal layer's set from the previous step; the set is refined
  at the first focal layer.
* same page, Methodology opening and Significance: the full cache is kept;
  only the attended subset changes per step.
* FastKV: Decoupling of Context Reduction and KV Cache Compression (section
  2A, Token-Selective Propagation): saliency is attention weight from a
  recent window of queries to all context tokens, averaged; the top-ranked
  tokens plus the window tokens are propagated.
* FastKV section 2B (Decoupled KV Retention): a KV budget per layer chosen
  independently of the propagation rate.
* FastKV section 2A, two-stage prefill: the layers after the TSP layer
  process only the propagated tokens (causal prefill over that sequence).
* HPD-Parsing wiki, method item 2 (shared-prefix KV reuse): branches read
  the shared visual context zero-copy and attend to it, their own layout
  prefix and their own history.

Readings where the pages are silent (each also listed with its reason in
the design notes): softmax scale 1/sqrt(d); q head h reads kv head
h // (Hq/Hkv); focal scores are softmax over the candidate segment, summed
over the head group (the window score instead normalises over every
visible key); window queries are causal; the average pool is zero-padded
and always divides by its width; ties go to the lower index; kept indices
are returned ascending.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def widen(x) -> np.ndarray:
    """bf16/fp32 tensor or array -> float64 ndarray (exact for bf16)."""
    if hasattr(x, "detach"):
        x = x.detach().float().cpu().numpy()
    return np.asarray(x, dtype=F64)


# ---------------------------------------------------------------------------
# KV store: logical rows of a paged cache
# ---------------------------------------------------------------------------

def logical_rows(pool, table_row, g: int, n: int, block: int = 16) -> np.ndarray:
    """Rows [0, n) of one sequence's kv head g from a paged pool.

    ``pool`` is [num_blocks][num_kv_heads][block][d]; logical row j lives in
    physical block table_row[j // block] at offset j % block.  A shared
    prefix is the same physical block ids in several tables, so reading it
    through any branch's table gives the same rows (HPD wiki, method item 2).
    """
    j = np.arange(n)
    tr = np.asarray(table_row, dtype=np.int64)
    blk = tr[j // block]
    off = j % block
    if hasattr(pool, "index_select"):
        import torch
        bt = torch.from_numpy(blk).to(pool.device)
        ot = torch.from_numpy(off).to(pool.device)
        return widen(pool[bt, g, ot, :])
    return widen(np.asarray(pool)[blk, g, off, :])


def fork_child_table(parent_table, parent_len: int, new_block: int, block: int = 16) -> np.ndarray:
    """A branch's block table at a fork.  HPD-Parsing wiki, inference
    scheduling: a content branch is spawned at a fork token and shares the
    parent's KV through a fork pointer, zero copy, released by reference
    count.  The blocks holding only rows before the fork point are shared as
    they are; a block the parent has only partly filled is replaced by
    new_block, a private copy, because both branches append after the fork
    point (copy on write).  Entries past the fork point are -1."""
    parent_table = np.asarray(parent_table, dtype=np.int64)
    t = np.full(parent_table.shape, -1, dtype=np.int64)
    nfull = parent_len // block
    t[:nfull] = parent_table[:nfull]
    if parent_len % block:
        t[nfull] = new_block
    return t


def copy_block(pool, src: int, dst: int) -> np.ndarray:
    """Pool with block dst replaced by a copy of block src (every kv head and
    row): the copy-on-write of a fork."""
    out = np.array(pool, copy=True)
    out[dst] = out[src]
    return out


# ---------------------------------------------------------------------------
# scoring
# ---------------------------------------------------------------------------

def logits(q, K, scale) -> np.ndarray:
    """s[..., j, i] = (q[..., j, :] . K[..., i, :]) * scale, in float64."""
    return (np.asarray(q, F64) @ np.swapaxes(np.asarray(K, F64), -1, -2)) * F64(scale)


def softmax(s) -> np.ndarray:
    s = np.asarray(s, F64)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def focal_scores(qg, K, s0: int, s1: int, scale, norm: str = "segment") -> np.ndarray:
    """Decode focal score of the candidate tokens [s0, s1) for one GQA group.

    qg: [..., G, d] the group's queries; K: [..., N, d] the group's logical
    K rows.  For each head: softmax of its logits over the candidate segment
    ("segment") or over all N rows read off at the segment ("context"),
    then the probabilities are summed over the G heads of the group.
    Result [..., s1 - s0], segment-relative (FastOCR, Focal-Guided Pruning).
    """
    s = logits(qg, K, scale)
    if norm == "segment":
        p = softmax(s[..., s0:s1])
    elif norm == "context":
        p = softmax(s)[..., s0:s1]
    else:
        raise ValueError(norm)
    return p.sum(axis=-2)


def window_scores(qw, K, s0: int, s1: int, scale, causal: bool = True) -> np.ndarray:
    """FastKV window saliency of tokens [s0, s1) for one GQA group.

    qw: [W, G, d], queries of the last W positions N-W .. N-1 (FastKV 2A:
    the queries of the most recent positions).  Each (window row, head) is a softmax
    over the keys it can see -- keys at positions <= its own when causal --
    and the probabilities are summed over the window rows and heads.
    """
    qw = np.asarray(qw, F64)
    K = np.asarray(K, F64)
    N = K.shape[0]
    W, G, d = qw.shape
    s = logits(qw.reshape(W * G, d), K, scale).reshape(W, G, N)   # every row's logits
    acc = np.zeros(N, F64)
    for r in range(W):
        pos = N - W + r
        vis = pos + 1 if causal else N
        p = softmax(s[r, :, :vis])                      # [G, vis]
        acc[:vis] += p.sum(axis=0)
    return acc[s0:s1]


def avg_pool(x, width: int) -> np.ndarray:
    """1-D average pool along the last axis, stride 1, 'same' length, zero
    padding; output i is the sum of the padded input over [i, i + width)
    divided by ``width`` (padding counted), width odd."""
    assert width % 2 == 1
    x = np.asarray(x, F64)
    h = width // 2
    zeros = np.zeros(x.shape[:-1] + (h,), F64)
    pad = np.concatenate([zeros, x, zeros], axis=-1)
    windows = np.lib.stride_tricks.sliding_window_view(pad, width, axis=-1)   # [..., n, width]
    return windows.sum(axis=-1) / width


# ---------------------------------------------------------------------------
# selection
# ---------------------------------------------------------------------------

def topk(scores, k: int) -> np.ndarray:
    """The k highest scores of each row (last axis); among equal float32
    scores the lower index wins.

    Full sort by (score descending, index ascending), keep the first k,
    return those indices ascending.
    """
    s32 = np.asarray(scores, dtype=np.float32).astype(F64)
    n = s32.shape[-1]
    if not 1 <= k <= n:
        raise ValueError("need 1 <= k <= n")
    order = np.lexsort((np.broadcast_to(np.arange(n), s32.shape), -s32), axis=-1)
    return np.sort(order[..., :k], axis=-1).astype(np.int64)


def topk_warm(scores, k: int, warm) -> np.ndarray:
    """Top-k restricted to candidates scoring at least theta, the lowest
    current score among the k warm indices (the previous step's set,
    FastOCR Cross-Step Fixation Reuse).  At least k candidates reach theta,
    so the k-th best score does too and the result is the top-k of the
    whole row."""
    s32 = np.asarray(scores, dtype=np.float32)
    warm = np.asarray(warm, dtype=np.int64)
    theta = s32[warm].min()
    cand = np.nonzero(s32 >= theta)[0]
    return cand[topk(s32[cand], k)]


def kept_rows(idx, s0: int, s1: int, n: int) -> np.ndarray:
    """Rows a sparse layer attends: the selected candidates (segment-relative
    idx shifted by s0) and every row outside the segment [s0, s1)."""
    idx = np.asarray(idx, dtype=np.int64)
    return np.concatenate([s0 + idx, np.arange(0, s0), np.arange(s1, n)])


def tie_band_check(gpu_idx, oracle_scores, k: int, rel: float = 1e-6):
    """Accept a kept set that may differ from the oracle's only at near ties.

    An index is ambiguous when its oracle score lies within ``rel`` of the
    k-th largest oracle score.  The kept set passes when it has k distinct
    in-range indices and every index in its symmetric difference with the
    oracle's set is ambiguous.  Returns (ok, n_diff) for one row
    (gpu_idx [k], oracle_scores [n]); for rows (gpu_idx [..., k],
    oracle_scores [..., n]) both are arrays over the rows (n_diff -1 for a
    row that is not k distinct in-range indices).
    """
    sc = np.asarray(oracle_scores, F64)
    g = np.asarray(gpu_idx, dtype=np.int64)
    n = sc.shape[-1]
    if g.shape[:-1] != sc.shape[:-1]:
        raise ValueError("gpu_idx must be [..., k] over the rows of oracle_scores")
    if g.shape[-1] != k:                                             # not k indices: every row fails
        return (False, -1) if g.ndim == 1 else (np.zeros(g.shape[:-1], bool), np.full(g.shape[:-1], -1))
    gs = np.sort(g, axis=-1)
    valid = (gs[..., 0] >= 0) & (gs[..., -1] < n) & np.all(gs[..., 1:] != gs[..., :-1], axis=-1)
    in_g = np.zeros(sc.shape, dtype=bool)
    np.put_along_axis(in_g, np.clip(g, 0, n - 1), True, axis=-1)
    in_o = np.zeros(sc.shape, dtype=bool)
    np.put_along_axis(in_o, topk(sc, k), True, axis=-1)
    sk = np.take(-np.sort(-sc, axis=-1), k - 1, axis=-1)           # k-th largest oracle score
    diff = in_g != in_o
    amb = np.abs(sc - sk[..., None]) <= rel * np.abs(sk)[..., None]
    ok = valid & np.all(~diff | amb, axis=-1)
    nd = np.where(valid, diff.sum(axis=-1), -1)
    if g.ndim == 1:
        return bool(ok), int(nd)
    return ok, nd


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def attention(qg, K, V, rows, scale):
    """Softmax attention of each query in qg [G, d] over the given rows of
    K, V ([N, d]).  Rows are taken as a set (ascending).  Returns
    (out [G, d], lse [G]) with lse the natural log of the softmax
    normaliser including the max shift."""
    r = np.unique(np.asarray(rows, dtype=np.int64))
    if r.shape[0] != np.asarray(rows).shape[0]:
        raise ValueError("rows must be distinct")
    Kr = np.asarray(K, F64)[r]
    Vr = np.asarray(V, F64)[r]
    s = logits(qg, Kr, scale)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    out = (e @ Vr) / z
    return out, (m + np.log(z))[:, 0]


def attention_masked(q, K, V, visible, scale):
    """Softmax attention of each query over the rows it may see: the same
    definition as ``attention`` with the row set given as a mask, so that
    many (sequence, head, step) instances go in one call.

    q [..., Q, d]; K, V [..., N, d]; visible: bool [..., Q, N] (or
    broadcastable to it), True where query j attends row i.  Returns
    (out [..., Q, d], lse [..., Q]); a query that sees no row gets out = 0
    and lse = -inf (FastOCR Cross-Layer Propagation: attention over the
    kept set only)."""
    s = logits(q, K, scale)
    vis = np.broadcast_to(np.asarray(visible, dtype=bool), s.shape)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    any_row = np.isfinite(m)
    m = np.where(any_row, m, 0.0)
    e = np.exp(s - m)                                   # exp(-inf) = 0 off the mask
    z = e.sum(axis=-1, keepdims=True)
    out = np.where(any_row, (e @ np.asarray(V, F64)) / np.where(any_row, z, 1.0), 0.0)
    lse = np.where(any_row, m + np.log(np.where(any_row, z, 1.0)), -np.inf)[..., 0]
    return out, lse


def verify_attention(qd, K, V, rows, n: int, scale):
    """Verification attention of m drafted tokens (HPD-Parsing wiki, P-MTP:
    each branch drafts several tokens and verifies them in parallel).

    qd: [m, G, d], the queries of the drafts at positions n-m .. n-1 (the
    drafts' own K/V rows are the last m rows).  Draft r attends over the
    rows of `rows` (the branch's attended set) at positions <= n-m+r:
    everything before the drafts, and the drafts up to its own (causal).
    Returns (out [m, G, d], lse [m, G])."""
    qd = np.asarray(qd, F64)
    m = qd.shape[0]
    r_all = np.unique(np.asarray(rows, dtype=np.int64))
    outs, lses = [], []
    for r in range(m):
        vis = r_all[r_all <= n - m + r]
        o, l = attention(qd[r], K, V, vis, scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def merge_attention(o1, lse1, o2, lse2):
    """Attention over the union of two disjoint row sets from the attention
    over each (out normalised per set, lse its log normaliser): the softmax
    normaliser of the union is the sum of the two, so each part is weighted
    by exp(lse_i - lse).  HPD-Parsing wiki, method item 2: a branch attends
    to the shared context and to its own rows, here computed apart and
    combined.  A part with no rows has lse = -inf and weight 0.
    o1, o2 [..., d]; lse1, lse2 [...].  Returns (out, lse)."""
    o1, o2 = np.asarray(o1, F64), np.asarray(o2, F64)
    l1, l2 = np.asarray(lse1, F64), np.asarray(lse2, F64)
    m = np.maximum(l1, l2)
    safe = np.where(np.isfinite(m), m, 0.0)
    w1, w2 = np.exp(l1 - safe), np.exp(l2 - safe)
    z = w1 + w2
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.where((z > 0)[..., None], (o1 * w1[..., None] + o2 * w2[..., None]) / np.where(z > 0, z, 1.0)[..., None], 0.0)
        lse = np.where(z > 0, safe + np.log(np.where(z > 0, z, 1.0)), -np.inf)
    return out, lse


def causal_prefill(Q, K, V, scale, rows=None):
    """Causal self-attention over the propagated tokens (FastKV, section 2A,
    Token-Selective Propagation: the layers after the TSP layer process only
    the top-ranked tokens and the window tokens).  The propagated tokens keep
    their order of position, so token i sees tokens 0..i.

    Q [n, hq, d]; K, V [n, hkv, d]; query head h reads kv head h // (hq/hkv).
    rows: (position, head) pairs to compute (default: every one, position
    major).  Returns (out [len(rows), d], lse [len(rows)])."""
    Q, K, V = np.asarray(Q, F64), np.asarray(K, F64), np.asarray(V, F64)
    n, hq = Q.shape[0], Q.shape[1]
    G = hq // K.shape[1]
    if rows is None:
        rows = [(i, h) for i in range(n) for h in range(hq)]
    outs, lses = [], []
    for i, h in rows:
        o, l = attention(Q[i, h][None], K[:, h // G], V[:, h // G], np.arange(i + 1), scale)
        outs.append(o[0])
        lses.append(l[0])
    return np.stack(outs), np.array(lses)


def dense_attention(qg, K, V, scale):
    return attention(qg, K, V, np.arange(np.asarray(K).shape[0]), scale)


def gather_rows(src, idx, tail_begin: int = 0, n_tail: int = 0):
    """Rows idx of src followed by rows [tail_begin, tail_begin + n_tail):
    the selected tokens' hidden states, then the window tokens
    (FastKV 2A: top-ranked tokens plus the window tokens)."""
    rows = np.concatenate([np.asarray(idx, dtype=np.int64),
                           np.arange(tail_begin, tail_begin + n_tail, dtype=np.int64)])
    return np.asarray(src)[rows]


# ---------------------------------------------------------------------------
# focal-layer profiling
# ---------------------------------------------------------------------------

def visual_mass(qg, K, s0: int, s1: int, scale) -> np.ndarray:
    """Image-attention ratio of each head of one GQA group: the share of the
    head's attention -- a softmax over all N rows -- that falls on the
    candidate (image) segment [s0, s1).  FastOCR, Focal-Guided Pruning,
    "Focal Layer Selection": the warm-up profiles every layer's
    image-attention ratio.  qg [G, d], K [N, d]; result [G]."""
    p = softmax(logits(qg, K, scale))
    return p[:, s0:s1].sum(axis=1)


def pick_focal_layers(ratios, n_pick: int) -> np.ndarray:
    """The focal layers: the n_pick layers whose image-attention ratio is
    highest on average (same page and section: a small fixed set of layers
    with high concentration on image tokens).

    ratios: [n_layers, n], each layer's ratios over the warm-up steps,
    sequences and heads.  The mean of each layer is taken exactly (a sum of
    rationals, so no rounding and no dependence on the order of the terms);
    a non-finite ratio counts as 0.  Layers ranked by mean descending, equal
    means to the lower layer; the first n_pick are returned ascending."""
    from fractions import Fraction
    r = np.asarray(ratios, F64)
    if not 1 <= n_pick <= r.shape[0]:
        raise ValueError("need 1 <= n_pick <= n_layers")
    n = r.shape[1]
    mean = [sum((Fraction(float(x)) for x in row if np.isfinite(x)), Fraction(0)) / n for row in r]
    order = sorted(range(r.shape[0]), key=lambda l: (-mean[l], l))
    return np.sort(np.asarray(order[:n_pick], dtype=np.int64))


# ---------------------------------------------------------------------------
# layer / step schedule
# ---------------------------------------------------------------------------

def focal_layer_plan(n_layers: int, focal, t: int):
    """What each layer does at decode step t.

    ('focal', l)               full attention + scoring + top-k
    ('sparse', l, ts, ls)      attend over the set chosen by layer ls at step ts
    ('dense', l)               full attention, no set to reuse yet

    Layers after a focal layer reuse the most recent focal layer's set of the
    same step (Cross-Layer Propagation).  Layers before the first focal layer
    reuse the deepest focal layer's set of step t-1 (Cross-Step Fixation
    Reuse); at t = 0 there is no previous step and they attend densely.
    """
    focal = sorted(set(int(f) for f in focal))
    first, last = focal[0], focal[-1]
    plan = []
    for l in range(n_layers):
        if l in focal:
            plan.append(("focal", l))
        elif l < first:
            plan.append(("dense", l) if t == 0 else ("sparse", l, t - 1, last))
        else:
            src = max(f for f in focal if f < l)
            plan.append(("sparse", l, t, src))
    return plan
