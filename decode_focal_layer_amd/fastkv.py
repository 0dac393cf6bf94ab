"""FastKV drivers over libkvsel calls (pointer passing only).

FastKV (section 2A, Token-Selective Propagation): at the TSP layer, the
window queries' attention weights over the prompt, summed over the window
rows and heads and smoothed by an average pool, rank the tokens; the top
ones plus the window tokens are propagated (their hidden states gathered).
Section 2B (Decoupled KV Retention): a per-kv-head decode budget chosen the
same way, then decode attends only to the retained rows plus the recent
rows and the rows generated since.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import torch

from . import kvsel


def tsp_select(kv: kvsel.KV, q_window: torch.Tensor, num_q_heads: int, scale: float, k: int, pool: int,
               hidden: Optional[torch.Tensor] = None, window: int = 8, causal: bool = True,
               scores: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
               dst: Optional[torch.Tensor] = None, ws: Optional[kvsel.Workspace] = None, stream=None):
    """One sequence's token-selective propagation: score (summed over all
    heads), top-k, and the gather of the selected rows of `hidden` followed by
    the window rows.  q_window: bf16 [1][window][hq][128]; hidden: [prompt][D]."""
    assert kv.batch == 1
    seg = kv.max_seg_len
    if scores is None:
        scores = torch.empty((1, 1, seg), dtype=torch.float32, device=q_window.device)
    if idx is None:
        idx = torch.empty((1, k), dtype=torch.int32, device=q_window.device)
    kvsel.score(kv, q_window, window, num_q_heads, scale, kvsel.REDUCE_ALL, kvsel.NORM_CONTEXT, causal, pool,
                scores, ws=ws, stream=stream)
    kvsel.topk(scores, seg, k, idx, stream=stream)
    if hidden is not None:
        if dst is None:
            dst = torch.empty((k + window, hidden.shape[1]), dtype=hidden.dtype, device=hidden.device)
        kvsel.gather_rows(hidden, idx, k, kv.max_seq_len - window, window, dst, stream=stream)
    return scores, idx, dst


class BudgetDecoder:
    """FastKV decode under a per-kv-head budget.  `kvs[p]` describes physical
    cache p (logical layer l reads cache l % len(kvs)).  select() chooses each
    cache's kept set once from its window queries; step() runs every logical
    layer's gathered attention for one decode step."""

    def __init__(self, kvs: Sequence[kvsel.KV], num_q_heads: int, k: int, layers: int, scale: float,
                 window: int = 8, pool: int = 7, device="cuda"):
        self.kvs = list(kvs)
        self.P = len(self.kvs)
        self.L = layers
        self.hq = num_q_heads
        self.k = k
        self.scale = float(scale)
        self.window = window
        self.pool = pool
        kv0 = self.kvs[0]
        self.B, self.hkv = kv0.batch, kv0.hkv
        seg = kv0.max_seg_len
        self.scores = torch.empty((self.B, self.hkv, seg), dtype=torch.float32, device=device)
        self.idx = [torch.empty((self.B, self.hkv, k), dtype=torch.int32, device=device) for _ in range(self.P)]
        self.out = torch.empty((layers, self.B, num_q_heads, 128), dtype=torch.float32, device=device)
        self.ws = kvsel.Workspace(device)

    def select(self, p: int, q_window: torch.Tensor, seq_len: torch.Tensor, stream=None):
        """q_window: bf16 [B][window][hq][128] of the last prompt positions."""
        kv = self.kvs[p].with_seq_len(seq_len)
        seg = kv.max_seg_len
        kvsel.score(kv, q_window, self.window, self.hq, self.scale, kvsel.REDUCE_GROUP, kvsel.NORM_CONTEXT, True,
                    self.pool, self.scores, ws=self.ws, stream=stream)
        kvsel.topk(self.scores, seg, self.k, self.idx[p], stream=stream)

    def step(self, q: torch.Tensor, seq_len: torch.Tensor, stream=None):
        """q: bf16 [layers][B][hq][128]; seq_len: int32 [B] (prompt + generated rows)."""
        for l in range(self.L):
            p = l % self.P
            kv = self.kvs[p]
            kv.c.seq_len = seq_len.data_ptr()
            kvsel.gather_attn(kv, q[l], self.hq, self.scale, self.idx[p], self.k, self.out[l], ws=self.ws,
                              stream=stream)
