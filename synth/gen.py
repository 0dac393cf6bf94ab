"""Seeded synthetic inputs for the five workloads.

Every tensor is drawn from its own torch generator whose seed is a hash of
(workload seed, tensor name, indices).  Values are i.i.d. N(0, 1) drawn in
fp32 and rounded to bf16 (round to nearest even, torch's conversion).
Structural draws (patch origins, step sizes, salient positions, suffix
lengths) come from numpy's Philox generator seeded the same way and are
made on the host, so they are identical on every device.

The fixation and salience constructions shape the inputs so that the
selection has something to find; they are part of the workload, not of the
method:

* key-side fixation (C0): the K rows of one 4x16 grid patch get
  ``boost * qhat_g`` added, qhat_g the unit vector of the group's summed
  query;
* query-side fixation (C1, C4): the cached K cannot change per step (it is
  reused across steps and, in C4, shared across branches), so the query of
  every head in group g gets ``boost * sqrt(d) * u_g`` added, u_g the unit
  vector of the summed K rows of the current patch;
* salient keys (C2, C3): ``boost * qhat_g`` added to K rows at seeded
  positions (C2) or in seeded 16-token clusters (C3), qhat_g the unit
  vector of the group's summed window queries.

The module holds none of the method's arithmetic: no logits, softmax,
scores, selection or attention.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

from .configs import BudgetDecode, FocalDecode, WindowSelect


def seed_of(*key) -> int:
    h = hashlib.blake2b(repr(key).encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def host_rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=seed_of(*key)))


def normal_bf16(shape, key, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(*key))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16)


def _unit(v: torch.Tensor) -> torch.Tensor:
    return v / v.norm(dim=-1, keepdim=True).clamp_min(1e-30)


def _ceil_div(a, b):
    return -(-a // b)


# --------------------------------------------------------------------------
# paged layout helpers (pure index bookkeeping)
# --------------------------------------------------------------------------

def contiguous_table(batch: int, blocks_per_seq: int) -> np.ndarray:
    """Block table where sequence b owns blocks [b*bps, (b+1)*bps)."""
    return (np.arange(batch, dtype=np.int64)[:, None] * blocks_per_seq
            + np.arange(blocks_per_seq, dtype=np.int64)[None, :]).astype(np.int32)


def shared_prefix_table(prefix_blocks: int, suffix_blocks: np.ndarray):
    """Block table where every branch maps its first ``prefix_blocks``
    logical blocks to the same physical blocks [0, prefix_blocks) and owns a
    private run of physical blocks for its suffix.  Unused entries are 0."""
    batch = len(suffix_blocks)
    maxb = prefix_blocks + int(suffix_blocks.max())
    table = np.zeros((batch, maxb), dtype=np.int32)
    table[:, :prefix_blocks] = np.arange(prefix_blocks, dtype=np.int32)[None, :]
    nxt = prefix_blocks
    for b in range(batch):
        n = int(suffix_blocks[b])
        table[b, prefix_blocks:prefix_blocks + n] = np.arange(nxt, nxt + n, dtype=np.int32)
        nxt += n
    return table, nxt


def patch_tokens(r: int, c: int, cols: int, ph: int, pw: int) -> np.ndarray:
    rr = np.arange(r, r + ph)[:, None]
    cc = np.arange(c, c + pw)[None, :]
    return (rr * cols + cc).reshape(-1)


def raster_walk(rows, cols, ph, pw, steps, start, deltas):
    """Patch origins along a raster reading order: move right by delta each
    step; wrap to column 0 and down one patch height at the right edge, and
    to row 0 at the bottom."""
    r, c = start
    out = []
    for t in range(steps):
        out.append((r, c))
        c += int(deltas[t])
        if c + pw > cols:
            c = 0
            r += ph
            if r + ph > rows:
                r = 0
    return out


def rows_to_physical(table: np.ndarray, b: int, tokens: np.ndarray, block: int):
    blk = table[b, tokens // block].astype(np.int64)
    return blk, (tokens % block).astype(np.int64)


# --------------------------------------------------------------------------
# FocalDecode workloads (C0, C1, C4)
# --------------------------------------------------------------------------

@dataclass
class FocalWorkload:
    cfg: FocalDecode
    k_pool: List[torch.Tensor]       # per layer: bf16 [num_blocks, hkv, block, d]
    v_pool: List[torch.Tensor]
    block_table: torch.Tensor        # int32 [B, max_blocks]
    q: torch.Tensor                  # bf16 [steps, layers, B, hq, d]
    seq_len: torch.Tensor            # int32 [steps, B]  rows present at step t
    seg_begin: torch.Tensor          # int32 [B]
    seg_end: torch.Tensor            # int32 [B]
    table_np: np.ndarray
    seq_len_np: np.ndarray           # [steps, B]
    patches: np.ndarray              # [steps, B, 2] patch origin (row, col) per step
    suffix_len: np.ndarray           # [B] (zeros unless shared-prefix)
    num_blocks: int
    max_blocks: int


def make_focal(cfg: FocalDecode, device="cpu") -> FocalWorkload:
    B, L, T = cfg.batch, cfg.layers, cfg.steps
    d, blk, hkv, hq, G = cfg.head_dim, cfg.block, cfg.hkv, cfg.hq, cfg.group
    ph, pw = cfg.patch
    appended = T if cfg.append else 0

    if cfg.shared_prefix:
        assert cfg.prefix_len % blk == 0
        lo, hi = cfg.suffix_range
        suffix = host_rng(cfg.seed, "suffix_len").integers(lo, hi + 1, size=B).astype(np.int64)
        sblocks = np.array([_ceil_div(int(s) + appended, blk) for s in suffix], dtype=np.int64)
        table, num_blocks = shared_prefix_table(cfg.prefix_len // blk, sblocks)
    else:
        suffix = np.zeros(B, dtype=np.int64)
        bps = _ceil_div(cfg.prefix_len + appended, blk)
        table = contiguous_table(B, bps)
        num_blocks = B * bps
    max_blocks = table.shape[1]

    seq_len = np.zeros((T, B), dtype=np.int32)
    for t in range(T):
        seq_len[t] = cfg.prefix_len + suffix + ((t + 1) if cfg.append else 0)

    # patch origins
    patches = np.zeros((T, B, 2), dtype=np.int64)
    for b in range(B):
        rng = host_rng(cfg.seed, "patch", b)
        start = (int(rng.integers(0, cfg.grid_rows - ph + 1)), int(rng.integers(0, cfg.grid_cols - pw + 1)))
        deltas = rng.integers(1, 3, size=T) if cfg.moving_patch else np.zeros(T, dtype=np.int64)
        patches[:, b, :] = np.array(raster_walk(cfg.grid_rows, cfg.grid_cols, ph, pw, T, start, deltas))

    k_pool, v_pool = [], []
    for l in range(L):
        k_pool.append(normal_bf16((num_blocks, hkv, blk, d), (cfg.seed, "K", l), device))
        v_pool.append(normal_bf16((num_blocks, hkv, blk, d), (cfg.seed, "V", l), device))
    q = torch.empty((T, L, B, hq, d), dtype=torch.bfloat16, device=device)
    for t in range(T):
        for l in range(L):
            q[t, l] = normal_bf16((B, hq, d), (cfg.seed, "Q", t, l), device)

    # physical coordinates of every patch token: [T, B, ph*pw]
    pblk = np.zeros((T, B, ph * pw), dtype=np.int64)
    poff = np.zeros((T, B, ph * pw), dtype=np.int64)
    for t in range(T):
        for b in range(B):
            toks = patch_tokens(int(patches[t, b, 0]), int(patches[t, b, 1]), cfg.grid_cols, ph, pw)
            pblk[t, b], poff[t, b] = rows_to_physical(table, b, toks, blk)
    pblk_t = torch.from_numpy(pblk).to(device)
    poff_t = torch.from_numpy(poff).to(device)

    if cfg.boost_side == "key":
        # C0: the patch (the same at every step) is written into K once.
        assert not cfg.moving_patch
        for l in range(L):
            qsum = q[0, l].float().view(B, hkv, G, d).sum(2)          # [B, hkv, d]
            qhat = _unit(qsum)
            for b in range(B):
                kb = k_pool[l][pblk_t[0, b], :, poff_t[0, b], :].float()  # [P, hkv, d]
                kb = kb + cfg.boost * qhat[b][None, :, :]
                k_pool[l][pblk_t[0, b], :, poff_t[0, b], :] = kb.to(torch.bfloat16)
    else:
        amp = cfg.boost * math.sqrt(d)
        for l in range(L):
            rows = k_pool[l][pblk_t, :, poff_t, :].float()              # [T, B, P, hkv, d]
            u = _unit(rows.sum(2))                                      # [T, B, hkv, d]
            qq = q[:, l].float().view(T, B, hkv, G, d) + amp * u[:, :, :, None, :]
            q[:, l] = qq.view(T, B, hq, d).to(torch.bfloat16)
            del rows, u, qq

    seg_begin = np.zeros(B, dtype=np.int32)
    seg_end = np.full(B, cfg.n_visual, dtype=np.int32)
    return FocalWorkload(
        cfg=cfg, k_pool=k_pool, v_pool=v_pool,
        block_table=torch.from_numpy(table).to(device),
        q=q, seq_len=torch.from_numpy(seq_len).to(device),
        seg_begin=torch.from_numpy(seg_begin).to(device),
        seg_end=torch.from_numpy(seg_end).to(device),
        table_np=table, seq_len_np=seq_len, patches=patches, suffix_len=suffix,
        num_blocks=num_blocks, max_blocks=max_blocks)


# --------------------------------------------------------------------------
# WindowSelect workload (C2)
# --------------------------------------------------------------------------

@dataclass
class WindowWorkload:
    cfg: WindowSelect
    k_pool: torch.Tensor       # bf16 [num_blocks, hkv, block, d]
    block_table: torch.Tensor  # int32 [B, max_blocks]
    q: torch.Tensor            # bf16 [B, W, hq, d]  queries of the last W positions
    hidden: Optional[torch.Tensor]   # bf16 [B*prompt, hidden]
    seq_len: torch.Tensor
    seg_begin: torch.Tensor
    seg_end: torch.Tensor
    salient: np.ndarray        # [B, n_salient] token positions
    table_np: np.ndarray
    num_blocks: int
    max_blocks: int


def make_window(cfg: WindowSelect, device="cpu", with_hidden=True) -> WindowWorkload:
    B, d, blk, hkv, hq, G, W = cfg.batch, cfg.head_dim, cfg.block, cfg.hkv, cfg.hq, cfg.group, cfg.window
    assert cfg.prompt % blk == 0
    bps = cfg.prompt // blk
    table = contiguous_table(B, bps)
    num_blocks = B * bps
    k_pool = normal_bf16((num_blocks, hkv, blk, d), (cfg.seed, "K"), device)
    q = normal_bf16((B, W, hq, d), (cfg.seed, "Qwin"), device)
    s0, s1 = cfg.seg
    salient = np.zeros((B, cfg.n_salient), dtype=np.int64)
    qhat = _unit(q.float().view(B, W, hkv, G, d).sum((1, 3)))          # [B, hkv, d]
    for b in range(B):
        pos = np.sort(host_rng(cfg.seed, "salient", b).choice(s1 - s0, size=cfg.n_salient, replace=False)) + s0
        salient[b] = pos
        pb, po = rows_to_physical(table, b, pos, blk)
        pb_t, po_t = torch.from_numpy(pb).to(device), torch.from_numpy(po).to(device)
        kk = k_pool[pb_t, :, po_t, :].float() + cfg.salient_boost * qhat[b][None]
        k_pool[pb_t, :, po_t, :] = kk.to(torch.bfloat16)
    hidden = normal_bf16((B * cfg.prompt, cfg.hidden), (cfg.seed, "hidden"), device) if with_hidden else None
    return WindowWorkload(
        cfg=cfg, k_pool=k_pool, block_table=torch.from_numpy(table).to(device), q=q, hidden=hidden,
        seq_len=torch.full((B,), cfg.prompt, dtype=torch.int32, device=device),
        seg_begin=torch.full((B,), s0, dtype=torch.int32, device=device),
        seg_end=torch.full((B,), s1, dtype=torch.int32, device=device),
        salient=salient, table_np=table, num_blocks=num_blocks, max_blocks=bps)


# --------------------------------------------------------------------------
# BudgetDecode workload (C3)
# --------------------------------------------------------------------------

@dataclass
class BudgetWorkload:
    cfg: BudgetDecode
    k_pool: List[torch.Tensor]     # per physical layer: bf16 [num_blocks, hkv, block, d]
    v_pool: List[torch.Tensor]
    block_table: torch.Tensor      # int32 [B, max_blocks]
    qwin: torch.Tensor             # bf16 [phys, B, W, hq, d] selection window queries
    q: torch.Tensor                # bf16 [steps, layers, B, hq, d] decode queries
    seq_len_sel: torch.Tensor      # int32 [B] = src_len
    seq_len: torch.Tensor          # int32 [steps, B] = src_len + t + 1
    seg_begin: torch.Tensor
    seg_end: torch.Tensor
    clusters: np.ndarray           # [phys, B, hkv, clusters] start positions
    table_np: np.ndarray
    num_blocks: int
    max_blocks: int


def make_budget(cfg: BudgetDecode, device="cpu") -> BudgetWorkload:
    B, d, blk, hkv, hq, G, W = cfg.batch, cfg.head_dim, cfg.block, cfg.hkv, cfg.hq, cfg.group, cfg.window
    P, T, L = cfg.phys_layers, cfg.steps, cfg.layers
    bps = _ceil_div(cfg.src_len + T, blk)
    table = contiguous_table(B, bps)
    num_blocks = B * bps
    s0, s1 = cfg.seg
    k_pool, v_pool = [], []
    qwin = torch.empty((P, B, W, hq, d), dtype=torch.bfloat16, device=device)
    clusters = np.zeros((P, B, hkv, cfg.clusters), dtype=np.int64)
    N = cfg.src_len
    for p in range(P):
        kp = normal_bf16((num_blocks, hkv, blk, d), (cfg.seed, "K", p), device)
        vp = normal_bf16((num_blocks, hkv, blk, d), (cfg.seed, "V", p), device)
        qw = normal_bf16((B, W, hq, d), (cfg.seed, "Qwin", p), device)
        qwin[p] = qw
        qhat = _unit(qw.float().view(B, W, hkv, G, d).sum((1, 3)))     # [B, hkv, d]
        for b in range(B):
            for g in range(hkv):
                # cluster [st, st + cluster_len) lies inside the candidate segment
                st = host_rng(cfg.seed, "cluster", p, b, g).integers(0, s1 - cfg.cluster_len + 1, size=cfg.clusters)
                clusters[p, b, g] = st
                toks = np.unique((st[:, None] + np.arange(cfg.cluster_len)[None, :]).reshape(-1))
                pb, po = rows_to_physical(table, b, toks, blk)
                pb_t, po_t = torch.from_numpy(pb).to(device), torch.from_numpy(po).to(device)
                kk = kp[pb_t, g, po_t, :].float() + cfg.salient_boost * qhat[b, g][None]
                kp[pb_t, g, po_t, :] = kk.to(torch.bfloat16)
        k_pool.append(kp)
        v_pool.append(vp)
    q = torch.empty((T, L, B, hq, d), dtype=torch.bfloat16, device=device)
    for t in range(T):
        for l in range(L):
            q[t, l] = normal_bf16((B, hq, d), (cfg.seed, "Q", t, l), device)
    seq_len = np.stack([np.full(B, N + t + 1, dtype=np.int32) for t in range(T)])
    return BudgetWorkload(
        cfg=cfg, k_pool=k_pool, v_pool=v_pool, block_table=torch.from_numpy(table).to(device),
        qwin=qwin, q=q,
        seq_len_sel=torch.full((B,), N, dtype=torch.int32, device=device),
        seq_len=torch.from_numpy(seq_len).to(device),
        seg_begin=torch.full((B,), s0, dtype=torch.int32, device=device),
        seg_end=torch.full((B,), s1, dtype=torch.int32, device=device),
        clusters=clusters, table_np=table, num_blocks=num_blocks, max_blocks=bps)
