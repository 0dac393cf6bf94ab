"""Decode-step driver: the focal-layer schedule over libkvsel calls.

FastOCR (technical summary, Focal-Guided Pruning / Cross-Layer Propagation):
only the focal layers attend over the full cache and select the top-k
visual tokens; every later layer attends over the most recent focal layer's
set.  Cross-Step Fixation Reuse: layers before the first focal layer reuse
the deepest focal layer's set from the previous step (at the first step
there is none and they attend densely); each focal layer's top-k is warm
started from its own previous selection.

This module only decides which buffer each call reads (index propagation
moves no data) and issues the calls; the arithmetic runs in the library.
The same driver serves the HPD-style branched decode: branches are the
sequences of the descriptor and share their prefix blocks through the
block table.
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import List, Optional, Sequence, Tuple

import torch

from . import kvsel


def shared_parts(query_rows: int, num_kv_heads: int, rows: int, per_cu: int = 1) -> int:
    """Parts to cut a shared row range into for kvsel_shared_attn: enough
    work-groups (one per 128 query rows of a kv head, per part) for per_cu
    per compute unit of a 256-CU device (two fit: with one, a part's tail
    overlaps the next work-group; the logits pass, whose stores leave the
    matrix cores idle, wants two), each part at least two 64-row tiles, at
    most 64 parts.  More parts cost a write and a read of each part's
    output."""
    groups = -(-query_rows // 128) * num_kv_heads
    want = -(-256 * per_cu // max(groups, 1))
    return max(1, min(want, 64, rows // 128))


def _cascade(L, own, kv, q, q_per_seq, hq, scale, rb, re, splits, parts_o, parts_lse, rows, out, lse_out,
             logits=None, ld_logits=0, stream=None):
    """One attention as the exact merge of a sequence's own rows and a shared
    row range [rb, re).  own(o, lse) enqueues the own-rows call writing
    there.  One part: own rows straight into out/lse_out, then the range
    folded in by kvsel_shared_attn (accumulate).  More: own rows in part 0,
    the range in parts 1 .. splits, one kvsel_merge_attn."""
    vp = ctypes.c_void_p
    lg = vp(logits.data_ptr()) if logits is not None else None
    if splits == 1:
        own(out, vp(lse_out.data_ptr()))
        kvsel._check(L.kvsel_shared_attn(kv.ref(), q, q_per_seq, hq, scale, rb, re, 1, 1, out,
                                         vp(lse_out.data_ptr()), lg, ld_logits, stream))
        return
    own(vp(parts_o[0].data_ptr()), vp(parts_lse[0].data_ptr()))
    kvsel._check(L.kvsel_shared_attn(kv.ref(), q, q_per_seq, hq, scale, rb, re, splits, 0,
                                     vp(parts_o[1].data_ptr()), vp(parts_lse[1].data_ptr()), lg, ld_logits, stream))
    kvsel._check(L.kvsel_merge_attn(vp(parts_o.data_ptr()), vp(parts_lse.data_ptr()), 1 + splits, rows, out,
                                    vp(lse_out.data_ptr()), stream))


class FocalDecoder:
    def __init__(self, kvs: Sequence[kvsel.KV], num_q_heads: int, k: int, focal: Sequence[int], scale: float,
                 seg_len: int, warm_start: bool = True, device="cuda", keep_scores: bool = False,
                 shared_tail: Optional[Tuple[int, int]] = None, shared_splits: Optional[int] = None):
        """shared_tail = (row_begin, row_end): every sequence's segment is
        [0, row_begin), and rows [0, row_end) are shared by all of them (the
        same cache blocks: HPD's visual and layout prefix).  Layers then attend
        in parts merged exactly (kvsel_merge_attn): each sequence's own rows
        by kvsel_gather_attn over a view whose segment reaches to row_end, and
        the shared rows once per kv head for all sequences by
        kvsel_shared_attn -- rows [row_begin, row_end) for sparse layers (in
        shared_splits parts, by default shared_parts' choice); the whole
        prefix for focal layers, whose segment logits then feed
        kvsel_select_logits."""
        self.kvs = list(kvs)
        self.L = len(self.kvs)
        self.hq = num_q_heads
        self.k = k
        self.focal = sorted(set(int(f) for f in focal))
        self.scale = float(scale)
        self.seg_len = seg_len
        self.warm_start = warm_start
        kv0 = self.kvs[0]
        B, hkv = kv0.batch, kv0.hkv
        self.B, self.hkv = B, hkv
        self.device = device
        self.keep_scores = keep_scores
        self.scores = torch.empty((B, hkv, seg_len), dtype=torch.float32, device=device) if keep_scores else None
        # two selection buffers per focal layer: this step's and the previous step's
        self.idx = {f: [torch.zeros((B, hkv, k), dtype=torch.int32, device=device) for _ in range(2)]
                    for f in self.focal}
        self.cur = 0
        self.out = torch.empty((self.L, B, num_q_heads, 128), dtype=torch.float32, device=device)
        self.ws = kvsel.Workspace(device)
        need = 0
        for kv in self.kvs:
            need = max(need, kvsel.attn_workspace(kv, num_q_heads, -1, True, kvsel.NORM_SEGMENT),
                       kvsel.attn_workspace(kv, num_q_heads, k))
        self.ws_ptr, self.ws_n = self.ws.ptr_and_size(need)
        self.t = 0
        self._lib = kvsel.lib()
        self.tail = None
        if shared_tail is not None:
            rb, re = int(shared_tail[0]), int(shared_tail[1])
            if not 0 <= rb <= re or any(re > kv.shared_rows for kv in self.kvs):
                raise ValueError("shared_tail must lie inside the shared rows")
            ext = torch.full((B,), re, dtype=torch.int32, device=device)
            # the private part: the segment reaches to row_end, so the shared rows are left out
            self.priv = [dataclasses.replace(kv, seg_end=ext, max_seg_len=kv.max_seg_len + (re - rb),
                                             min_seg_len=kv.min_seg_len + (re - rb)) for kv in self.kvs]
            self.tail = (rb, re)
            G = num_q_heads // hkv
            self.splits = int(shared_splits) if shared_splits is not None else shared_parts(B * G, hkv, re - rb)
            self.focal_splits = shared_parts(B * G, hkv, re, per_cu=2)
            # part 0: each sequence's own rows; parts 1 ..: the shared rows (one part is folded in place)
            np_ = 1 + max(self.splits, self.focal_splits)
            self.parts_o = self.parts_lse = None
            if np_ > 2:
                self.parts_o = torch.empty((np_, B, num_q_heads, 128), dtype=torch.float32, device=device)
                self.parts_lse = torch.empty((np_, B, num_q_heads), dtype=torch.float32, device=device)
            self.lse_out = torch.empty((B, num_q_heads), dtype=torch.float32, device=device)
            self.logits = torch.empty((B, num_q_heads, seg_len), dtype=torch.float32, device=device)

    def plan(self, t: int):
        """(kind, src_step_is_previous, src_layer) per layer."""
        first, last = self.focal[0], self.focal[-1]
        plan = []
        for l in range(self.L):
            if l in self.focal:
                plan.append(("focal", None))
            elif l < first:
                plan.append(("dense", None) if t == 0 else ("sparse", ("prev", last)))
            else:
                plan.append(("sparse", ("cur", max(f for f in self.focal if f < l))))
        return plan

    def step(self, t: int, q: torch.Tensor, seq_len: torch.Tensor, stream=None, layer_hook=None):
        """One decode step.  q: bf16 [layers][B][hq][128]; seq_len: int32 [B]
        (rows present, including this step's appended row)."""
        L = self._lib
        st = kvsel._stream(stream)
        cur, prev = self.cur, 1 - self.cur
        sl = seq_len.data_ptr()
        for l, (kind, src) in enumerate(self.plan(t)):
            kv = self.kvs[l]
            kv.c.seq_len = sl
            qp = ctypes.c_void_p(q[l].data_ptr())
            op = ctypes.c_void_p(self.out[l].data_ptr())
            if layer_hook is not None:
                layer_hook(l, kind, "begin")
            if kind == "focal" and self.tail is not None:
                warm = self.idx[l][prev].data_ptr() if (self.warm_start and t > 0) else None
                pk = self.priv[l]
                pk.c.seq_len = sl

                def own(o, ls, pk=pk):   # own rows (after the prefix): no kept rows, the segment view covers the prefix
                    kvsel._check(L.kvsel_gather_attn(pk.ref(), qp, self.hq, self.scale, None, 0, o, ls,
                                                     self.ws_ptr, self.ws_n, st))
                _cascade(L, own, kv, qp, 1, self.hq, self.scale, 0, self.tail[1], self.focal_splits, self.parts_o,
                         self.parts_lse, self.B * self.hq, op, self.lse_out, self.logits, self.seg_len, st)
                lg = ctypes.c_void_p(self.logits.data_ptr())
                kvsel._check(L.kvsel_select_logits(kv.ref(), lg, self.seg_len, self.hq, self.scale,
                                                   kvsel.NORM_SEGMENT, self.k, warm,
                                                   ctypes.c_void_p(self.idx[l][cur].data_ptr()), self.scores_ptr(),
                                                   self.seg_len if self.keep_scores else 0, st))
            elif kind == "focal":
                warm = self.idx[l][prev].data_ptr() if (self.warm_start and t > 0) else None
                kvsel._check(L.kvsel_focal_attn(kv.ref(), qp, self.hq, self.scale, op, None, kvsel.NORM_SEGMENT,
                                                self.k, warm, ctypes.c_void_p(self.idx[l][cur].data_ptr()),
                                                self.scores_ptr(), self.seg_len if self.keep_scores else 0,
                                                self.ws_ptr, self.ws_n, st))
            elif kind == "dense":
                kvsel._check(L.kvsel_dense_attn(kv.ref(), qp, self.hq, self.scale, op, None, None, 0,
                                                kvsel.NORM_SEGMENT, self.ws_ptr, self.ws_n, st))
            else:
                which, ls = src
                buf = self.idx[ls][cur if which == "cur" else prev]
                if self.tail is None:
                    kvsel._check(L.kvsel_gather_attn(kv.ref(), qp, self.hq, self.scale,
                                                     ctypes.c_void_p(buf.data_ptr()), self.k, op, None,
                                                     self.ws_ptr, self.ws_n, st))
                else:
                    pk = self.priv[l]
                    pk.c.seq_len = sl

                    def own(o, ls, pk=pk, buf=buf):
                        kvsel._check(L.kvsel_gather_attn(pk.ref(), qp, self.hq, self.scale,
                                                         ctypes.c_void_p(buf.data_ptr()), self.k, o, ls,
                                                         self.ws_ptr, self.ws_n, st))
                    _cascade(L, own, kv, qp, 1, self.hq, self.scale, self.tail[0], self.tail[1], self.splits,
                             self.parts_o, self.parts_lse, self.B * self.hq, op, self.lse_out, stream=st)
            if layer_hook is not None:
                layer_hook(l, kind, "end")
        self.cur = prev   # this step's selection becomes "previous"

    def scores_ptr(self):
        return ctypes.c_void_p(self.scores.data_ptr()) if self.keep_scores else None

    def selection(self, layer: int, previous: bool = False) -> torch.Tensor:
        """Kept indices of a focal layer after the last step (or the step before)."""
        return self.idx[layer][self.cur if previous else 1 - self.cur]


class FocalProfiler:
    """Warm-up profiling and the choice of the focal layers.

    FastOCR (technical summary, Focal-Guided Pruning, "Focal Layer
    Selection"): during w warm-up steps every layer's image-attention ratio
    is profiled, and the small fixed set of layers that concentrate most on
    the image tokens becomes the focal set.  Each step writes each layer's
    per-(sequence, head) ratios (kvsel_visual_mass) into that layer's row of
    one buffer; pick() ranks the layers by mean ratio (kvsel_pick_layers).
    """

    def __init__(self, kvs: Sequence[kvsel.KV], num_q_heads: int, scale: float, warmup_steps: int, device="cuda"):
        self.kvs = list(kvs)
        self.L = len(self.kvs)
        self.hq = num_q_heads
        self.scale = float(scale)
        self.w = int(warmup_steps)
        self.B = self.kvs[0].batch
        self.per_step = self.B * num_q_heads
        self.ratios = torch.zeros((self.L, self.w * self.per_step), dtype=torch.float32, device=device)
        self.ws = kvsel.Workspace(device)
        need = max(kvsel.lib().kvsel_mass_workspace(kv.ref(), num_q_heads) for kv in self.kvs)
        self.ws.ptr_and_size(need)
        self.layers = torch.zeros((self.L,), dtype=torch.int32, device=device)

    def step(self, t: int, q: torch.Tensor, seq_len: torch.Tensor, stream=None):
        """Warm-up step t < w; q: bf16 [layers][batch][hq][128]."""
        if not 0 <= t < self.w:
            raise ValueError("warm-up step out of range")
        for l, kv in enumerate(self.kvs):
            kv.c.seq_len = seq_len.data_ptr()
            kvsel.visual_mass(kv, q[l], self.hq, self.scale,
                              self.ratios[l, t * self.per_step:(t + 1) * self.per_step], ws=self.ws, stream=stream)

    def pick(self, n_focal: int, stream=None) -> torch.Tensor:
        """The n_focal layers with the highest mean ratio, ascending (int32, device)."""
        return kvsel.pick_layers(self.ratios, n_focal, self.layers[:n_focal], stream=stream)


class DraftVerifier:
    """Verification attention of m drafts per sequence (HPD-Parsing wiki,
    P-MTP) over one layer's cache.  With shared_tail = (row_begin, row_end)
    -- every sequence's segment ends at row_begin and rows [row_begin,
    row_end) are the same cache blocks in every table -- it runs as a
    cascade: each sequence's own rows (kvsel_verify_attn with the segment
    extended to row_end), the shared rows once per kv head for every draft of
    every sequence (kvsel_shared_attn), merged exactly: folded into the
    output in place when the range is one part (the default for many
    queries), else by kvsel_merge_attn."""

    def __init__(self, kv: kvsel.KV, m: int, num_q_heads: int, scale: float,
                 shared_tail: Optional[Tuple[int, int]] = None, shared_splits: Optional[int] = None,
                 device="cuda"):
        self.kv, self.m, self.hq, self.scale = kv, int(m), num_q_heads, float(scale)
        B = kv.batch
        self.tail = None
        if shared_tail is not None:
            rb, re = int(shared_tail[0]), int(shared_tail[1])
            if not 0 <= rb <= re or re > kv.shared_rows:
                raise ValueError("shared_tail must lie inside the shared rows")
            ext = torch.full((B,), re, dtype=torch.int32, device=device)
            self.priv = dataclasses.replace(kv, seg_end=ext, max_seg_len=kv.max_seg_len + (re - rb),
                                            min_seg_len=kv.min_seg_len + (re - rb))
            self.tail = (rb, re)
            G = num_q_heads // kv.hkv
            self.splits = (int(shared_splits) if shared_splits is not None
                           else shared_parts(B * self.m * G, kv.hkv, re - rb))
            self.parts_o = self.parts_lse = None   # one part is folded in place
            if self.splits > 1:
                self.parts_o = torch.empty((1 + self.splits, B, self.m, num_q_heads, 128), dtype=torch.float32,
                                           device=device)
                self.parts_lse = torch.empty((1 + self.splits, B, self.m, num_q_heads), dtype=torch.float32,
                                             device=device)
            self.lse_out = torch.empty((B, self.m, num_q_heads), dtype=torch.float32, device=device)

    def verify(self, q: torch.Tensor, idx: Optional[torch.Tensor], k: int, out: torch.Tensor,
               lse: Optional[torch.Tensor] = None, stream=None):
        """q: bf16 [B][m][hq][128]; out: fp32 [B][m][hq][128]."""
        if self.tail is None:
            return kvsel.verify_attn(self.kv, q, self.m, self.hq, self.scale, idx, k, out, lse, stream=stream)
        L = kvsel.lib()
        st = kvsel._stream(stream)
        self.priv.c.seq_len = self.kv.c.seq_len
        qp = ctypes.c_void_p(q.data_ptr())

        def own(o, ls):
            kvsel._check(L.kvsel_verify_attn(self.priv.ref(), qp, self.m, self.hq, self.scale,
                                             ctypes.c_void_p(idx.data_ptr()) if idx is not None else None, k, o, ls,
                                             st))
        _cascade(L, own, self.kv, qp, self.m, self.hq, self.scale, self.tail[0], self.tail[1], self.splits,
                 self.parts_o, self.parts_lse, self.kv.batch * self.m * self.hq, ctypes.c_void_p(out.data_ptr()),
                 lse if lse is not None else self.lse_out, stream=st)
        return out
