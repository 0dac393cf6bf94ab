"""Python binding of libkvsel (ctypes).

Argument marshalling only: tensors become raw device pointers, the current
torch stream becomes the hipStream_t, a non-zero status becomes KvselError.
Every step of the path runs in the library's HIP kernels; nothing here
computes.  PyTorch supplies device memory and streams.

The binding fails loudly if libkvsel.so has not been built.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# the library built in-tree; KVSEL_LIBRARY names another build of the same
# sources (the host-sanitizer build the CPU tests load)
LIB_PATH = os.environ.get("KVSEL_LIBRARY") or os.path.join(_HERE, "libkvsel.so")

REDUCE_GROUP, REDUCE_ALL = 0, 1
NORM_SEGMENT, NORM_CONTEXT = 0, 1
FLAG_DETERMINISTIC = 1
STATUS = {0: "KVSEL_OK", -1: "KVSEL_EINVAL", -2: "KVSEL_ENOSPC", -3: "KVSEL_EUNSUPPORTED", -4: "KVSEL_EHIP",
          -5: "KVSEL_EDEBUG"}

# every symbol the public header declares
SYMBOLS = (
    "kvsel_version", "kvsel_status_string", "kvsel_last_error", "kvsel_debug_status",
    "kvsel_score", "kvsel_score_workspace",
    "kvsel_topk", "kvsel_topk_workspace",
    "kvsel_gather_attn", "kvsel_attn_workspace", "kvsel_gather_attn_noalloc",
    "kvsel_dense_attn", "kvsel_focal_attn", "kvsel_gather_rows",
    "kvsel_visual_mass", "kvsel_mass_workspace", "kvsel_pick_layers",
    "kvsel_pool_create", "kvsel_pool_destroy", "kvsel_pool_free_count", "kvsel_pool_refcount",
    "kvsel_pool_alloc", "kvsel_pool_retain", "kvsel_pool_release", "kvsel_fork",
    "kvsel_verify_attn", "kvsel_prefill_attn", "kvsel_shared_attn", "kvsel_merge_attn", "kvsel_select_logits",
)


class KvselError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class KvDescC(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
        ("max_seg_len", ctypes.c_int32), ("min_seg_len", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64),
        ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("seq_len", ctypes.c_void_p),
        ("seg_begin", ctypes.c_void_p), ("seg_end", ctypes.c_void_p),
        ("shared_rows", ctypes.c_int32), ("flags", ctypes.c_int32),
    ]


_lib: Optional[ctypes.CDLL] = None
_P = ctypes.c_void_p
_DP = ctypes.POINTER(KvDescC)
_I32, _I64, _F32, _SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """Load libkvsel.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libkvsel.so not found at {LIB_PATH}: build it with "
                           "`python -m decode_focal_layer_amd.build` (there is no fallback path)")
    L = ctypes.CDLL(LIB_PATH)
    L.kvsel_version.restype = _I32
    L.kvsel_status_string.restype = ctypes.c_char_p
    L.kvsel_status_string.argtypes = [_I32]
    L.kvsel_last_error.restype = ctypes.c_char_p
    L.kvsel_debug_status.restype = _I32
    L.kvsel_debug_status.argtypes = [_P, _P, _P]
    L.kvsel_score.restype = _I32
    L.kvsel_score.argtypes = [_DP, _P, _I32, _I32, _F32, _I32, _I32, _I32, _I32, _P, _I64, _P, _SZ, _P]
    L.kvsel_score_workspace.restype = _SZ
    L.kvsel_score_workspace.argtypes = [_DP, _I32, _I32, _I32, _I32]
    L.kvsel_topk.restype = _I32
    L.kvsel_topk.argtypes = [_P, _I64, _I32, _P, _I32, _I32, _P, _P, _P, _SZ, _P]
    L.kvsel_topk_workspace.restype = _SZ
    L.kvsel_topk_workspace.argtypes = [_I32, _I32, _I32]
    L.kvsel_gather_attn.restype = _I32
    L.kvsel_gather_attn.argtypes = [_DP, _P, _I32, _F32, _P, _I32, _P, _P, _P, _SZ, _P]
    L.kvsel_gather_attn_noalloc.restype = _I32
    L.kvsel_gather_attn_noalloc.argtypes = [_DP, _P, _I32, _F32, _P, _I32, _P, _P, _P]
    L.kvsel_attn_workspace.restype = _SZ
    L.kvsel_attn_workspace.argtypes = [_DP, _I32, _I32, _I32, _I32]
    L.kvsel_dense_attn.restype = _I32
    L.kvsel_dense_attn.argtypes = [_DP, _P, _I32, _F32, _P, _P, _P, _I64, _I32, _P, _SZ, _P]
    L.kvsel_focal_attn.restype = _I32
    L.kvsel_focal_attn.argtypes = [_DP, _P, _I32, _F32, _P, _P, _I32, _I32, _P, _P, _P, _I64, _P, _SZ, _P]
    L.kvsel_gather_rows.restype = _I32
    L.kvsel_gather_rows.argtypes = [_P, _I64, _I64, _P, _I32, _I64, _I32, _P, _P]
    L.kvsel_visual_mass.restype = _I32
    L.kvsel_visual_mass.argtypes = [_DP, _P, _I32, _F32, _P, _P, _SZ, _P]
    L.kvsel_mass_workspace.restype = _SZ
    L.kvsel_mass_workspace.argtypes = [_DP, _I32]
    L.kvsel_pick_layers.restype = _I32
    L.kvsel_pick_layers.argtypes = [_P, _I64, _I32, _I32, _I32, _P, _P]
    L.kvsel_pool_create.restype = _P
    L.kvsel_pool_create.argtypes = [_I64]
    L.kvsel_pool_destroy.restype = None
    L.kvsel_pool_destroy.argtypes = [_P]
    L.kvsel_pool_free_count.restype = _I64
    L.kvsel_pool_free_count.argtypes = [_P]
    L.kvsel_pool_refcount.restype = _I32
    L.kvsel_pool_refcount.argtypes = [_P, _I32]
    for fn in (L.kvsel_pool_alloc, L.kvsel_pool_retain, L.kvsel_pool_release):
        fn.restype = _I32
        fn.argtypes = [_P, _P, _I32] if fn is not L.kvsel_pool_alloc else [_P, _I32, _P]
    L.kvsel_verify_attn.restype = _I32
    L.kvsel_verify_attn.argtypes = [_DP, _P, _I32, _I32, _F32, _P, _I32, _P, _P, _P]
    L.kvsel_shared_attn.restype = _I32
    L.kvsel_shared_attn.argtypes = [_DP, _P, _I32, _I32, _F32, _I32, _I32, _I32, _I32, _P, _P, _P, ctypes.c_int64,
                                    _P]
    L.kvsel_select_logits.restype = _I32
    L.kvsel_select_logits.argtypes = [_DP, _P, ctypes.c_int64, _I32, _F32, _I32, _I32, _P, _P, _P, ctypes.c_int64, _P]
    L.kvsel_merge_attn.restype = _I32
    L.kvsel_merge_attn.argtypes = [_P, _P, _I32, ctypes.c_int64, _P, _P, _P]
    L.kvsel_prefill_attn.restype = _I32
    L.kvsel_prefill_attn.argtypes = [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _F32, _P, _P, _P]
    L.kvsel_fork.restype = _I32
    L.kvsel_fork.argtypes = [_P, _P, _I32, _I32, _P, _P, _P, _I64, _I32, _P]
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise KvselError(status, lib().kvsel_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ---------------------------------------------------------------------------
# descriptor and workspace
# ---------------------------------------------------------------------------

@dataclass
class KV:
    """A paged KV cache view.  Keeps the tensors alive while the C struct
    holds their addresses."""
    k_pool: torch.Tensor
    v_pool: Optional[torch.Tensor]
    block_table: torch.Tensor
    seq_len: torch.Tensor
    seg_begin: torch.Tensor
    seg_end: torch.Tensor
    max_seq_len: int
    max_seg_len: int
    min_seg_len: int = 0
    shared_rows: int = 0   # cache hint: leading rows shared across sequences
    deterministic: bool = False   # KVSEL_FLAG_DETERMINISTIC: bitwise reproducible attention

    def __post_init__(self):
        _need(self.k_pool, torch.bfloat16, "k_pool")
        if self.v_pool is not None:
            _need(self.v_pool, torch.bfloat16, "v_pool")
            if self.v_pool.shape != self.k_pool.shape:
                raise ValueError("k_pool and v_pool shapes differ")
        for n in ("block_table", "seq_len", "seg_begin", "seg_end"):
            _need(getattr(self, n), torch.int32, n)
        nb, hkv, blk, d = self.k_pool.shape
        c = KvDescC()
        c.batch = self.block_table.shape[0]
        c.num_kv_heads = hkv
        c.head_dim = d
        c.block_size = blk
        c.max_blocks_per_seq = self.block_table.shape[1]
        c.max_seq_len = int(self.max_seq_len)
        c.max_seg_len = int(self.max_seg_len)
        c.min_seg_len = int(self.min_seg_len)
        c.num_blocks = nb
        c.k_pool = self.k_pool.data_ptr()
        c.v_pool = self.v_pool.data_ptr() if self.v_pool is not None else None
        c.block_table = self.block_table.data_ptr()
        c.seq_len = self.seq_len.data_ptr()
        c.seg_begin = self.seg_begin.data_ptr()
        c.seg_end = self.seg_end.data_ptr()
        c.shared_rows = int(self.shared_rows)
        c.flags = FLAG_DETERMINISTIC if self.deterministic else 0
        self.c = c

    @property
    def batch(self):
        return self.c.batch

    @property
    def hkv(self):
        return self.c.num_kv_heads

    def ref(self):
        return ctypes.byref(self.c)

    def with_seq_len(self, seq_len: torch.Tensor, max_seq_len: Optional[int] = None) -> "KV":
        return KV(self.k_pool, self.v_pool, self.block_table, seq_len, self.seg_begin, self.seg_end,
                  self.max_seq_len if max_seq_len is None else max_seq_len, self.max_seg_len, self.min_seg_len,
                  self.shared_rows, self.deterministic)


class Workspace:
    """Zero-filled device scratch, grown on demand (a grown buffer is zero-filled
    again; the library leaves its counters at zero after every call)."""

    def __init__(self, device="cuda", nbytes: int = 0):
        self.device = device
        self.buf = None
        if nbytes:
            self.ensure(nbytes)

    def ensure(self, nbytes: int) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.zeros(max(nbytes, 256) + 256, dtype=torch.uint8, device=self.device)
        return self.buf

    def ptr_and_size(self, nbytes: int):
        b = self.ensure(nbytes)
        addr = b.data_ptr()
        pad = (-addr) % 256
        return ctypes.c_void_p(addr + pad), b.numel() - pad


_default_ws = {}


def _ws(ws: Optional[Workspace], device) -> Workspace:
    if ws is not None:
        return ws
    key = str(device)
    if key not in _default_ws:
        _default_ws[key] = Workspace(device)
    return _default_ws[key]


# ---------------------------------------------------------------------------
# entry points (same names as the C calls)
# ---------------------------------------------------------------------------

def version() -> int:
    return lib().kvsel_version()


def debug_status():
    """kvsel_debug_status: (status, violations, first code, first detail).  A
    release build gives KVSEL_EUNSUPPORTED; synchronise the device first."""
    n, c, d = ctypes.c_uint32(0), ctypes.c_uint32(0), ctypes.c_uint32(0)
    st = lib().kvsel_debug_status(ctypes.byref(n), ctypes.byref(c), ctypes.byref(d))
    return st, n.value, c.value, d.value


def score_workspace(kv: KV, n_rows: int, num_q_heads: int, reduce: int, norm: int) -> int:
    return lib().kvsel_score_workspace(kv.ref(), n_rows, num_q_heads, reduce, norm)


def attn_workspace(kv: KV, num_q_heads: int, k: int, with_scores: bool = False, norm: int = NORM_SEGMENT) -> int:
    return lib().kvsel_attn_workspace(kv.ref(), num_q_heads, k, int(with_scores), norm)


def score(kv: KV, q: torch.Tensor, n_rows: int, num_q_heads: int, scale: float, reduce: int, norm: int,
          causal: bool, pool_width: int, scores: torch.Tensor, ws: Optional[Workspace] = None, stream=None):
    """kvsel_score.  q: bf16 [batch][n_rows][hq][128]; scores: fp32 [batch][hkv or 1][ld]."""
    _need(q, torch.bfloat16, "q")
    _need(scores, torch.float32, "scores")
    w = _ws(ws, q.device)
    p, n = w.ptr_and_size(score_workspace(kv, n_rows, num_q_heads, reduce, norm))
    _check(lib().kvsel_score(kv.ref(), _ptr(q), n_rows, num_q_heads, scale, reduce, norm, int(causal),
                             pool_width, _ptr(scores), scores.shape[-1], p, n, _stream(stream)))
    return scores


def topk_workspace(rows: int, n: int, k: int) -> int:
    return lib().kvsel_topk_workspace(rows, n, k)


def topk(scores: torch.Tensor, n: int, k: int, idx: torch.Tensor, warm: Optional[torch.Tensor] = None,
         n_per_row: Optional[torch.Tensor] = None, ws: Optional[Workspace] = None, stream=None):
    """kvsel_topk.  scores: fp32 [..., ld] viewed as rows; idx: int32 [rows][k];
    n_per_row: int32 [rows] candidate counts (each clamped to n) or None."""
    _need(scores, torch.float32, "scores")
    _need(idx, torch.int32, "idx")
    ld = scores.shape[-1]
    rows = scores.numel() // ld
    if idx.numel() != rows * k:
        raise ValueError("idx must hold rows * k entries")
    if warm is not None:
        _need(warm, torch.int32, "warm")
        if warm.numel() != rows * k:
            raise ValueError("warm must hold rows * k entries")
    if n_per_row is not None:
        _need(n_per_row, torch.int32, "n_per_row")
        if n_per_row.numel() != rows:
            raise ValueError("n_per_row must hold one count per row")
    w = _ws(ws, scores.device)
    p, nb = w.ptr_and_size(topk_workspace(rows, n, k))
    _check(lib().kvsel_topk(_ptr(scores), ld, rows, _ptr(n_per_row), n, k, _ptr(warm), _ptr(idx), p, nb,
                            _stream(stream)))
    return idx


def gather_attn(kv: KV, q: torch.Tensor, num_q_heads: int, scale: float, idx: Optional[torch.Tensor], k: int,
                out: torch.Tensor, lse: Optional[torch.Tensor] = None, ws: Optional[Workspace] = None,
                stream=None):
    """kvsel_gather_attn.  q: bf16 [batch][hq][128]; idx: int32 [batch][hkv][k]; out fp32 [batch][hq][128]."""
    _need(q, torch.bfloat16, "q")
    _need(out, torch.float32, "out")
    if idx is not None:
        _need(idx, torch.int32, "idx")
        if idx.numel() != kv.batch * kv.hkv * k:
            raise ValueError("idx must be [batch][num_kv_heads][k]")
    if lse is not None:
        _need(lse, torch.float32, "lse")
    w = _ws(ws, q.device)
    p, n = w.ptr_and_size(attn_workspace(kv, num_q_heads, k))
    _check(lib().kvsel_gather_attn(kv.ref(), _ptr(q), num_q_heads, scale, _ptr(idx), k, _ptr(out), _ptr(lse),
                                   p, n, _stream(stream)))
    return out


def gather_attn_noalloc(kv: KV, q: torch.Tensor, num_q_heads: int, scale: float, idx: Optional[torch.Tensor],
                        k: int, out: torch.Tensor, lse: Optional[torch.Tensor] = None, stream=None):
    """kvsel_gather_attn_noalloc: kvsel_gather_attn with the library's fixed
    per-device scratch instead of a workspace (no allocation anywhere)."""
    _need(q, torch.bfloat16, "q")
    _need(out, torch.float32, "out")
    if idx is not None:
        _need(idx, torch.int32, "idx")
        if idx.numel() != kv.batch * kv.hkv * k:
            raise ValueError("idx must be [batch][num_kv_heads][k]")
    if lse is not None:
        _need(lse, torch.float32, "lse")
    _check(lib().kvsel_gather_attn_noalloc(kv.ref(), _ptr(q), num_q_heads, scale, _ptr(idx), k, _ptr(out),
                                           _ptr(lse), _stream(stream)))
    return out


def dense_attn(kv: KV, q: torch.Tensor, num_q_heads: int, scale: float, out: torch.Tensor,
               lse: Optional[torch.Tensor] = None, seg_scores: Optional[torch.Tensor] = None,
               norm: int = NORM_SEGMENT, ws: Optional[Workspace] = None, stream=None):
    """kvsel_dense_attn, optionally fused with the focal scores [batch][hkv][ld]."""
    _need(q, torch.bfloat16, "q")
    _need(out, torch.float32, "out")
    if lse is not None:
        _need(lse, torch.float32, "lse")
    ld = 0
    if seg_scores is not None:
        _need(seg_scores, torch.float32, "seg_scores")
        ld = seg_scores.shape[-1]
    w = _ws(ws, q.device)
    p, n = w.ptr_and_size(attn_workspace(kv, num_q_heads, -1, seg_scores is not None, norm))
    _check(lib().kvsel_dense_attn(kv.ref(), _ptr(q), num_q_heads, scale, _ptr(out), _ptr(lse), _ptr(seg_scores),
                                  ld, norm, p, n, _stream(stream)))
    return out


def verify_attn(kv: KV, q: torch.Tensor, m: int, num_q_heads: int, scale: float, idx: Optional[torch.Tensor], k: int,
                out: torch.Tensor, lse: Optional[torch.Tensor] = None, stream=None):
    """kvsel_verify_attn.  q: bf16 [batch][m][hq][128]; out: fp32 [batch][m][hq][128]."""
    _need(q, torch.bfloat16, "q")
    _need(out, torch.float32, "out")
    if idx is not None:
        _need(idx, torch.int32, "idx")
    if lse is not None:
        _need(lse, torch.float32, "lse")
    _check(lib().kvsel_verify_attn(kv.ref(), _ptr(q), m, num_q_heads, scale, _ptr(idx), k, _ptr(out), _ptr(lse),
                                   _stream(stream)))
    return out


def prefill_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int,
                 scale: float, out: torch.Tensor, lse: Optional[torch.Tensor] = None, stream=None):
    """kvsel_prefill_attn.  q: bf16 [total][hq][128]; k, v: bf16 [total][hkv][128];
    cu_seqlens: int32 [batch + 1]; out: fp32 [total][hq][128]."""
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, name)
    _need(cu_seqlens, torch.int32, "cu_seqlens")
    _need(out, torch.float32, "out")
    if lse is not None:
        _need(lse, torch.float32, "lse")
    if q.dim() != 3 or k.dim() != 3 or k.shape != v.shape or q.shape[0] != k.shape[0]:
        raise ValueError("q [total, hq, 128], k and v [total, hkv, 128]")
    _check(lib().kvsel_prefill_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), cu_seqlens.numel() - 1, max_seqlen,
                                    q.shape[1], k.shape[1], scale, _ptr(out), _ptr(lse), _stream(stream)))
    return out


def shared_attn(kv: KV, q: torch.Tensor, num_q_heads: int, scale: float, row_begin: int, row_end: int,
                out: torch.Tensor, lse: Optional[torch.Tensor] = None, splits: int = 1, q_per_seq: int = 1,
                logits: Optional[torch.Tensor] = None, accumulate: bool = False, stream=None):
    """kvsel_shared_attn.  q: bf16 [batch][q_per_seq][hq][128]; out: fp32
    [splits][batch][q_per_seq][hq][128]; lse: fp32 [splits][batch][q_per_seq][hq];
    logits: fp32 [batch][hq][ld] (segment rows' raw dots) or None;
    accumulate: out/lse hold another part on entry and get this range merged in."""
    _need(q, torch.bfloat16, "q")
    _need(out, torch.float32, "out")
    if lse is not None:
        _need(lse, torch.float32, "lse")
    if logits is not None:
        _need(logits, torch.float32, "logits")
    _check(lib().kvsel_shared_attn(kv.ref(), _ptr(q), q_per_seq, num_q_heads, scale, row_begin, row_end, splits,
                                   int(bool(accumulate)), _ptr(out), _ptr(lse), _ptr(logits), logits.shape[-1] if logits is not None else 0,
                                   _stream(stream)))
    return out


def select_logits(kv: KV, logits: torch.Tensor, num_q_heads: int, scale: float, k: int, idx: torch.Tensor,
                  warm: Optional[torch.Tensor] = None, seg_scores: Optional[torch.Tensor] = None, stream=None):
    """kvsel_select_logits.  logits: fp32 [batch][hq][ld]; idx: int32 [batch][hkv][k]."""
    _need(logits, torch.float32, "logits")
    _need(idx, torch.int32, "idx")
    _check(lib().kvsel_select_logits(kv.ref(), _ptr(logits), logits.shape[-1], num_q_heads, scale, NORM_SEGMENT, k,
                                     _ptr(warm), _ptr(idx), _ptr(seg_scores),
                                     seg_scores.shape[-1] if seg_scores is not None else 0, _stream(stream)))
    return idx


def merge_attn(o: torch.Tensor, lse: torch.Tensor, out: torch.Tensor, lse_out: torch.Tensor, stream=None):
    """kvsel_merge_attn.  o: fp32 [parts][rows..][128]; lse: fp32 [parts][rows..];
    out: fp32 [rows..][128]; lse_out: fp32 [rows..] (out may be a part of o)."""
    for t, name in ((o, "o"), (lse, "lse"), (out, "out"), (lse_out, "lse_out")):
        _need(t, torch.float32, name)
    parts = lse.shape[0]
    rows = lse[0].numel()
    if o.numel() != parts * rows * 128 or out.numel() != rows * 128 or lse_out.numel() != rows:
        raise ValueError("o: [parts][rows][128]; lse: [parts][rows]; out: [rows][128]; lse_out: [rows]")
    _check(lib().kvsel_merge_attn(_ptr(o), _ptr(lse), parts, rows, _ptr(out), _ptr(lse_out), _stream(stream)))
    return out


def visual_mass(kv: KV, q: torch.Tensor, num_q_heads: int, scale: float, mass: torch.Tensor,
                ws: Optional[Workspace] = None, stream=None):
    """kvsel_visual_mass.  q: bf16 [batch][hq][128]; mass: fp32, batch * hq
    contiguous values (e.g. a slice of a per-layer ratio buffer)."""
    _need(q, torch.bfloat16, "q")
    _need(mass, torch.float32, "mass")
    if mass.numel() < kv.batch * num_q_heads:
        raise ValueError("mass needs batch * num_q_heads values")
    w = _ws(ws, q.device)
    p, n = w.ptr_and_size(lib().kvsel_mass_workspace(kv.ref(), num_q_heads))
    _check(lib().kvsel_visual_mass(kv.ref(), _ptr(q), num_q_heads, scale, _ptr(mass), p, n, _stream(stream)))
    return mass


def pick_layers(ratios: torch.Tensor, n_pick: int, layers: torch.Tensor, stream=None):
    """kvsel_pick_layers.  ratios: fp32 [n_layers][n] (row stride = its
    second dimension); layers: int32 [n_pick]."""
    _need(ratios, torch.float32, "ratios")
    _need(layers, torch.int32, "layers")
    if ratios.dim() != 2 or layers.numel() < n_pick:
        raise ValueError("ratios must be [n_layers][n] and layers hold n_pick values")
    _check(lib().kvsel_pick_layers(_ptr(ratios), ratios.shape[1], ratios.shape[0], ratios.shape[1], n_pick,
                                   _ptr(layers), _stream(stream)))
    return layers


def focal_attn(kv: KV, q: torch.Tensor, num_q_heads: int, scale: float, out: torch.Tensor, k: int,
               idx: torch.Tensor, warm: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
               seg_scores: Optional[torch.Tensor] = None, norm: int = NORM_SEGMENT,
               ws: Optional[Workspace] = None, stream=None):
    """kvsel_focal_attn: dense attention + focal scores + top-k per (sequence, kv head).
    idx (and warm): int32 [batch][hkv][k]."""
    _need(q, torch.bfloat16, "q")
    _need(out, torch.float32, "out")
    _need(idx, torch.int32, "idx")
    if idx.numel() != kv.batch * kv.hkv * k:
        raise ValueError("idx must be [batch][num_kv_heads][k]")
    if warm is not None:
        _need(warm, torch.int32, "warm")
        if warm.numel() != idx.numel():
            raise ValueError("warm must be [batch][num_kv_heads][k]")
    if lse is not None:
        _need(lse, torch.float32, "lse")
    ld = 0
    if seg_scores is not None:
        _need(seg_scores, torch.float32, "seg_scores")
        ld = seg_scores.shape[-1]
    w = _ws(ws, q.device)
    p, n = w.ptr_and_size(attn_workspace(kv, num_q_heads, -1, True, norm))
    _check(lib().kvsel_focal_attn(kv.ref(), _ptr(q), num_q_heads, scale, _ptr(out), _ptr(lse), norm, k, _ptr(warm),
                                  _ptr(idx), _ptr(seg_scores), ld, p, n, _stream(stream)))
    return idx


def gather_rows(src: torch.Tensor, idx: Optional[torch.Tensor], n_idx: int, tail_begin: int, n_tail: int,
                dst: torch.Tensor, stream=None):
    """kvsel_gather_rows: dst = src[idx[:n_idx]] ++ src[tail_begin : tail_begin + n_tail] (rows)."""
    if not src.is_contiguous() or not dst.is_contiguous():
        raise ValueError("src and dst must be contiguous")
    row_bytes = math.prod(src.shape[1:]) * src.element_size()
    if idx is not None:
        _need(idx, torch.int32, "idx")
    _check(lib().kvsel_gather_rows(_ptr(src), row_bytes, src.shape[0], _ptr(idx), n_idx, tail_begin, n_tail,
                                   _ptr(dst), _stream(stream)))
    return dst


# ---------------------------------------------------------------------------
# branch lifecycle

class BlockPool:
    """kvsel_block_pool: reference-counted physical block ids of one paged
    cache (host side), and the fork of a branch (kvsel_fork)."""

    def __init__(self, num_blocks: int):
        self._p = lib().kvsel_pool_create(int(num_blocks))
        if not self._p:
            raise ValueError("num_blocks must be in [1, 2^31)")
        self.num_blocks = int(num_blocks)

    def __del__(self):
        if getattr(self, "_p", None):
            lib().kvsel_pool_destroy(self._p)
            self._p = None

    @staticmethod
    def _ids(ids):
        import numpy as np
        a = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
        return a, a.ctypes.data_as(ctypes.c_void_p)

    def free_count(self) -> int:
        return lib().kvsel_pool_free_count(self._p)

    def refcount(self, block: int) -> int:
        return lib().kvsel_pool_refcount(self._p, int(block))

    def alloc(self, n: int):
        import numpy as np
        a = np.zeros(max(n, 1), dtype=np.int32)
        _check(lib().kvsel_pool_alloc(self._p, int(n), a.ctypes.data_as(ctypes.c_void_p)))
        return a[:n]

    def retain(self, ids):
        a, p = self._ids(ids)
        _check(lib().kvsel_pool_retain(self._p, p, a.shape[0]))

    def release(self, ids):
        a, p = self._ids(ids)
        _check(lib().kvsel_pool_release(self._p, p, a.shape[0]))

    def fork(self, parent_table, parent_len: int, k_pool: Optional[torch.Tensor] = None,
             v_pool: Optional[torch.Tensor] = None, stream=None):
        """The child's block table (numpy int32, like parent_table).  A
        partly filled last block is copied on the device (k_pool, v_pool:
        the cache's bf16 pools)."""
        import numpy as np
        pt = np.ascontiguousarray(np.asarray(parent_table, dtype=np.int32))
        ct = np.full_like(pt, -1)
        nb, hkv = (k_pool.shape[0], k_pool.shape[1]) if k_pool is not None else (self.num_blocks, 0)
        st = _stream(stream) if k_pool is not None else None
        _check(lib().kvsel_fork(self._p, pt.ctypes.data_as(ctypes.c_void_p), int(parent_len), pt.shape[0],
                                ct.ctypes.data_as(ctypes.c_void_p), _ptr(k_pool), _ptr(v_pool), nb, hkv, st))
        return ct
