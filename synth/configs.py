"""Workload definitions: the five synthetic workloads as plain data.

Each workload is shaped like one of the settings the pages describe:

* ``C0`` one FastOCR decode step (FastOCR technical summary, "Focal-Guided
  Pruning": top-attended image tokens at kept ratio tau; "Experimental
  Results": 5% of visual tokens).
* ``C1`` a multi-step FastOCR decode with focal layers and cross-step
  fixation reuse (FastOCR, "Cross-Layer Propagation" and "Cross-Step
  Fixation Reuse").
* ``C2`` the FastKV token-selective propagation layer (FastKV section 2A):
  window-averaged attention weights rank the prompt, the top-ranked tokens
  plus the window tokens are propagated.
* ``C3`` FastKV decode under a compressed per-head KV budget (FastKV
  section 2B, decoupled KV retention).
* ``C4`` HPD-style branched decode over a zero-copy shared prefix (HPD
  wiki, method item 2, shared-prefix KV reuse and context isolation; the
  backbone shape from the page header: 28 layers, 16 q / 8 kv heads).

No formula is printed on the pages for the score; the readings taken here
(softmax scale 1/sqrt(d), consecutive GQA grouping, segment or context
normalisation, lowest-index tie-break, rounding of the budget) are data
fields below so that every consumer reads the same value.

This module holds shapes and knobs only: no arithmetic of the method.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

HEAD_DIM = 128
BLOCK = 16


def budget(ratio: float, base: int) -> int:
    """Kept count from a ratio: round half up of ratio*base.

    The pages give budgets as ratios (5% of visual tokens in FastOCR; a
    TSP rate in FastKV 2B).  Rounding to nearest is the one rule that gives
    179 for 5% of 3584 and 6554 for 20% of a 32768-token prompt.
    """
    return int(math.floor(ratio * base + 0.5))


@dataclass(frozen=True)
class FocalDecode:
    """Decode with focal layers (C0, C1, C4).

    Tokens of the visual grid are row-major, token = r * grid_cols + c, and
    occupy positions [0, grid_rows*grid_cols) of every sequence; the
    ``n_always`` text/layout rows follow; decode appends one row per step.
    """
    name: str
    seed: int
    layers: int
    batch: int
    hq: int
    hkv: int
    grid_rows: int
    grid_cols: int
    n_always: int                 # text (C0, C1) or layout (C4) rows after the grid
    steps: int
    focal: Tuple[int, ...]
    tau: float = 0.05
    patch: Tuple[int, int] = (4, 16)
    boost: float = 0.5
    boost_side: str = "query"     # "key": K rows of the patch += boost*qhat; "query": see synth.gen
    moving_patch: bool = True
    shared_prefix: bool = False   # C4: one prefix referenced by every branch's block table
    suffix_range: Optional[Tuple[int, int]] = None   # C4: per-branch suffix length U[lo, hi]
    append: bool = True           # one new row per step is attended (decode appends)
    warm_start: bool = True
    head_dim: int = HEAD_DIM
    block: int = BLOCK

    @property
    def n_visual(self) -> int:
        return self.grid_rows * self.grid_cols

    @property
    def prefix_len(self) -> int:
        return self.n_visual + self.n_always

    @property
    def k(self) -> int:
        return budget(self.tau, self.n_visual)

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


@dataclass(frozen=True)
class WindowSelect:
    """FastKV token-selective propagation at one layer (C2)."""
    name: str
    seed: int
    batch: int
    hq: int
    hkv: int
    prompt: int
    window: int = 8
    pool: int = 7
    rate: float = 0.2
    n_salient: int = 256
    salient_boost: float = 0.4
    hidden: int = 4096
    causal: bool = True
    head_dim: int = HEAD_DIM
    block: int = BLOCK

    @property
    def seg(self) -> Tuple[int, int]:
        return (0, self.prompt - self.window)

    @property
    def k(self) -> int:
        return budget(self.rate, self.prompt)

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


@dataclass(frozen=True)
class BudgetDecode:
    """FastKV decode under a per-kv-head budget (C3).

    ``layers`` logical layers alias ``phys_layers`` physical caches:
    logical layer l reads cache l % phys_layers.  Selection runs once per
    physical cache with its own window queries.
    """
    name: str
    seed: int
    batch: int
    layers: int
    phys_layers: int
    hq: int
    hkv: int
    src_len: int
    budget: int = 2048
    recent: int = 64
    window: int = 8
    pool: int = 7
    steps: int = 128
    clusters: int = 128
    cluster_len: int = 16
    salient_boost: float = 0.4
    causal: bool = True
    head_dim: int = HEAD_DIM
    block: int = BLOCK

    @property
    def seg(self) -> Tuple[int, int]:
        return (0, self.src_len - self.recent)

    @property
    def k(self) -> int:
        return self.budget

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


C0 = FocalDecode(name="c0_single_step", seed=20260000, layers=1, batch=1, hq=16, hkv=8,
                 grid_rows=56, grid_cols=64, n_always=512, steps=1, focal=(0,),
                 boost_side="key", moving_patch=False, append=False, warm_start=False)

C1 = FocalDecode(name="c1_fastocr_decode", seed=20260001, layers=28, batch=32, hq=16, hkv=8,
                 grid_rows=80, grid_cols=80, n_always=1024, steps=64, focal=(3, 14))

C2 = WindowSelect(name="c2_fastkv_tsp", seed=20260002, batch=1, hq=32, hkv=8, prompt=32768)

C3 = BudgetDecode(name="c3_fastkv_budget_decode", seed=20260003, batch=16, layers=32,
                  phys_layers=8, hq=32, hkv=8, src_len=131072)

C4 = FocalDecode(name="c4_hpd_branched", seed=20260004, layers=28, batch=512, hq=16, hkv=8,
                 grid_rows=48, grid_cols=64, n_always=1024, steps=32, focal=(3, 14),
                 shared_prefix=True, suffix_range=(32, 1024))

CONFIGS = {"c0": C0, "c1": C1, "c2": C2, "c3": C3, "c4": C4}


def small(cfg, **kw):
    """A reduced copy of a workload for fast parity runs (same structure)."""
    return replace(cfg, **kw)
