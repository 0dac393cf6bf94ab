"""The C-ABI library loads, exports every symbol its header declares, and
rejects bad arguments on the host before any HIP call (so these run without
a GPU: a call that reached HIP would return KVSEL_EHIP instead of the code
asserted here)."""
import ctypes
import os
import re

import pytest

from decode_focal_layer_amd import kvsel

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "kvsel.h")
EINVAL, ENOSPC, EUNSUP = -1, -2, -3
FAKE = 1 << 20        # a 256-byte aligned address that is never dereferenced on the host


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(kvsel.LIB_PATH):
        from decode_focal_layer_amd import build
        build.build()
    return kvsel.lib()


def declared():
    txt = open(HDR).read()
    return sorted(set(re.findall(r"KVSEL_API\s+[\w\s\*]*?\b(kvsel_\w+)\s*\(", txt)))


def test_exports_every_declared_symbol(L):
    names = declared()
    assert len(names) == 30
    assert sorted(kvsel.SYMBOLS) == names
    for n in names:
        assert hasattr(L, n), n
    assert L.kvsel_version() == 3
    assert L.kvsel_status_string(-2) == b"workspace too small"
    assert L.kvsel_status_string(-5) == b"device check failed"


def desc(**over):
    d = kvsel.KvDescC()
    vals = dict(batch=2, num_kv_heads=8, head_dim=128, block_size=16, max_blocks_per_seq=10, max_seq_len=150,
                max_seg_len=100, min_seg_len=100, num_blocks=20, k_pool=FAKE, v_pool=FAKE + 4096,
                block_table=FAKE, seq_len=FAKE, seg_begin=FAKE, seg_end=FAKE)
    vals.update(over)
    for k, v in vals.items():
        setattr(d, k, v)
    return d


def gather(L, d, hq=16, q=FAKE, k=5, idx=FAKE, out=FAKE, ws=FAKE, ws_bytes=1 << 30, scale=0.088):
    return L.kvsel_gather_attn(ctypes.byref(d), q, hq, scale, idx, k, out, None, ws, ws_bytes, None)


@pytest.mark.parametrize("over,code", [
    (dict(head_dim=64), EUNSUP), (dict(block_size=32), EUNSUP), (dict(batch=0), EINVAL),
    (dict(num_kv_heads=0), EINVAL), (dict(max_blocks_per_seq=0), EINVAL), (dict(max_seq_len=161), EINVAL),
    (dict(max_seg_len=151), EINVAL), (dict(min_seg_len=101), EINVAL), (dict(num_blocks=0), EINVAL),
    (dict(k_pool=0), EINVAL), (dict(v_pool=0), EINVAL), (dict(block_table=0), EINVAL), (dict(seq_len=0), EINVAL),
    (dict(seg_begin=0), EINVAL), (dict(seg_end=0), EINVAL), (dict(k_pool=FAKE + 8), EINVAL),
    (dict(batch=4096, num_kv_heads=8), EUNSUP), (dict(num_blocks=1 << 28), EUNSUP),
    (dict(shared_rows=-1), EINVAL), (dict(flags=2), EINVAL), (dict(flags=-1), EINVAL),
])
def test_gather_attn_rejects_bad_descriptor(L, over, code):
    assert gather(L, desc(**over)) == code
    assert L.kvsel_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(hq=12), EINVAL), (dict(hq=72), EUNSUP), (dict(hq=0), EINVAL), (dict(q=0), EINVAL),
    (dict(q=FAKE + 2), EINVAL), (dict(out=0), EINVAL), (dict(k=-1), EINVAL), (dict(idx=0), EINVAL),
    (dict(scale=float("inf")), EINVAL), (dict(ws=0), EINVAL), (dict(ws=FAKE + 64), EINVAL),
    (dict(ws_bytes=64), ENOSPC),
])
def test_gather_attn_rejects_bad_args(L, kw, code):
    assert gather(L, desc(), **kw) == code


def test_gather_attn_noalloc_rejects(L):
    """The allocation-free variant validates like kvsel_gather_attn, and a
    call needing more split records than its fixed 4 MiB buffer holds is
    refused with KVSEL_ENOSPC before anything is enqueued."""
    na = lambda d, hq=16, k=5, idx=FAKE, out=FAKE: L.kvsel_gather_attn_noalloc(ctypes.byref(d), FAKE, hq, 0.088, idx, k,
                                                                                out, None, None)
    assert na(desc(head_dim=64)) == EUNSUP
    assert na(desc(), hq=12) == EINVAL
    assert na(desc(), out=0) == EINVAL
    assert na(desc(), k=-1) == EINVAL
    assert na(desc(), idx=0) == EINVAL
    # 64 x 8 pairs of G = 8 split in two: 64 * 64 * 2 records of 640 B > 4 MiB
    big = desc(batch=64, max_blocks_per_seq=100, max_seq_len=1600, max_seg_len=1000, min_seg_len=1000, num_blocks=6400)
    assert na(big, hq=64) == ENOSPC
    assert b"fixed buffer" in L.kvsel_last_error()


def test_dense_attn_checks(L):
    d = desc()
    r = L.kvsel_dense_attn(ctypes.byref(d), FAKE, 16, 0.088, FAKE, None, FAKE, 99, 0, FAKE, 1 << 30, None)
    assert r == EINVAL          # ld < max_seg_len
    r = L.kvsel_dense_attn(ctypes.byref(d), FAKE, 16, 0.088, FAKE, None, FAKE, 100, 7, FAKE, 1 << 30, None)
    assert r == EINVAL          # bad norm
    r = L.kvsel_dense_attn(ctypes.byref(d), FAKE, 16, 0.088, FAKE, None, FAKE, 100, 0, FAKE, 16, None)
    assert r == ENOSPC
    need = L.kvsel_attn_workspace(ctypes.byref(d), 16, -1, 1, 0)
    assert need > L.kvsel_attn_workspace(ctypes.byref(d), 16, -1, 0, 0) > 0
    assert L.kvsel_attn_workspace(ctypes.byref(desc(head_dim=64)), 16, -1, 0, 0) == 0


def test_focal_attn_checks(L):
    d = desc()
    f = lambda dd, **kw: L.kvsel_focal_attn(ctypes.byref(dd), kw.get("q", FAKE), 16, 0.088, FAKE, None, kw.get("norm", 0),
                                            kw.get("k", 5), None, kw.get("idx", FAKE), kw.get("sc", None),
                                            kw.get("ld", 0), FAKE, kw.get("ws_bytes", 1 << 30), None)
    assert f(d, k=0) == EINVAL
    assert f(d, idx=0) == EINVAL
    assert f(d, norm=3) == EINVAL
    assert f(d, sc=FAKE, ld=50) == EINVAL
    assert f(d, ws_bytes=100) == ENOSPC
    big = desc(max_blocks_per_seq=1000, max_seq_len=16000, max_seg_len=12289, min_seg_len=0, num_blocks=4000)
    assert f(big) == EUNSUP


def score(L, d, q=FAKE, n_rows=1, hq=16, reduce=0, norm=0, causal=1, pool=1, scores=FAKE, ld=100,
          ws=FAKE, ws_bytes=1 << 30):
    return L.kvsel_score(ctypes.byref(d), q, n_rows, hq, 0.088, reduce, norm, causal, pool, scores, ld, ws,
                         ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(n_rows=0), EINVAL), (dict(n_rows=65), EINVAL), (dict(reduce=2), EINVAL), (dict(norm=2), EINVAL),
    (dict(n_rows=8, norm=0), EINVAL), (dict(n_rows=8, norm=1, hq=72), EUNSUP), (dict(pool=2), EINVAL),
    (dict(pool=0), EINVAL), (dict(ld=99), EINVAL), (dict(scores=0), EINVAL), (dict(q=0), EINVAL),
    (dict(ws_bytes=8), ENOSPC), (dict(n_rows=8, norm=1, ws_bytes=8), ENOSPC),
])
def test_score_rejects(L, kw, code):
    assert score(L, desc(v_pool=0), **kw) == code


def test_score_workspace_sizes(L):
    d = desc(v_pool=0)
    assert L.kvsel_score_workspace(ctypes.byref(d), 1, 16, 0, 0) > 0
    assert L.kvsel_score_workspace(ctypes.byref(d), 8, 32, 1, 1) > 0
    assert L.kvsel_score_workspace(ctypes.byref(d), 0, 16, 0, 0) == 0


@pytest.mark.parametrize("args,code", [
    (dict(scores=0), EINVAL), (dict(idx=0), EINVAL), (dict(rows=0), EINVAL), (dict(k=0), EINVAL),
    (dict(k=11, n=10), EINVAL), (dict(n=20, ld=10), EINVAL),
])
def test_topk_rejects(L, args, code):
    a = dict(scores=FAKE, ld=10, rows=4, n=10, k=3, warm=None, idx=FAKE)
    a.update(args)
    assert L.kvsel_topk(a["scores"], a["ld"], a["rows"], None, a["n"], a["k"], a["warm"], a["idx"], None, 0,
                        None) == code
    assert L.kvsel_topk_workspace(4, 10, 3) == 0


def test_topk_long_rows_need_a_workspace(L):
    """Rows too long to stage in LDS (more than 36864 candidates) take the
    two-kernel path, whose per-slice coarse counts (2048 per 8192-key slice
    of each row) live in the workspace."""
    assert L.kvsel_topk_workspace(2, 40000, 10) == 2 * 5 * 2048 * 4
    assert L.kvsel_topk_workspace(2, 36864, 10) == 0
    assert L.kvsel_topk_workspace(2, 40000, 0) == 0
    t = lambda ws, nb: L.kvsel_topk(FAKE, 40000, 2, None, 40000, 10, None, FAKE, ws, nb, None)
    assert t(None, 0) == EINVAL
    assert t(FAKE + 64, 1 << 20) == EINVAL
    assert t(FAKE, 1000) == ENOSPC
    assert L.kvsel_topk(FAKE, 10, 70000, None, 10, 3, None, FAKE, None, 0, None) == EINVAL   # rows > 65535


@pytest.mark.parametrize("args,code", [
    (dict(src=0), EINVAL), (dict(dst=0), EINVAL), (dict(src=FAKE + 4), EINVAL), (dict(row_bytes=24), EINVAL),
    (dict(row_bytes=0), EINVAL), (dict(n_idx=-1), EINVAL), (dict(n_tail=-1), EINVAL), (dict(idx=0), EINVAL),
])
def test_gather_rows_rejects(L, args, code):
    a = dict(src=FAKE, row_bytes=8192, n_src=100, idx=FAKE, n_idx=5, tail=90, n_tail=3, dst=FAKE)
    a.update(args)
    r = L.kvsel_gather_rows(a["src"], a["row_bytes"], a["n_src"], a["idx"], a["n_idx"], a["tail"], a["n_tail"],
                            a["dst"], None)
    assert r == code


@pytest.mark.parametrize("kw,code", [
    (dict(hq=12), EINVAL), (dict(q=0), EINVAL), (dict(q=FAKE + 2), EINVAL), (dict(mass=0), EINVAL),
    (dict(scale=float("nan")), EINVAL), (dict(ws_bytes=16), ENOSPC), (dict(ws=0), EINVAL),
    (dict(d=dict(head_dim=64)), EUNSUP), (dict(d=dict(k_pool=0)), EINVAL),
])
def test_visual_mass_rejects(L, kw, code):
    d = desc(v_pool=0, **kw.get("d", {}))    # V is never read: v_pool may be NULL
    r = L.kvsel_visual_mass(ctypes.byref(d), kw.get("q", FAKE), kw.get("hq", 16), kw.get("scale", 0.088),
                            kw.get("mass", FAKE), kw.get("ws", FAKE), kw.get("ws_bytes", 1 << 30), None)
    assert r == code
    assert L.kvsel_last_error()


def test_mass_workspace(L):
    assert L.kvsel_mass_workspace(ctypes.byref(desc(v_pool=0)), 16) > 0
    assert L.kvsel_mass_workspace(ctypes.byref(desc(head_dim=64)), 16) == 0


@pytest.mark.parametrize("args,code", [
    (dict(ratios=0), EINVAL), (dict(layers=0), EINVAL), (dict(n_layers=0), EINVAL), (dict(n_layers=1025), EINVAL),
    (dict(n=0), EINVAL), (dict(ld=3), EINVAL), (dict(n_pick=0), EINVAL), (dict(n_pick=29), EINVAL),
])
def test_pick_layers_rejects(L, args, code):
    a = dict(ratios=FAKE, ld=64, n_layers=28, n=64, n_pick=2, layers=FAKE)
    a.update(args)
    assert L.kvsel_pick_layers(a["ratios"], a["ld"], a["n_layers"], a["n"], a["n_pick"], a["layers"], None) == code


@pytest.mark.parametrize("kw,code", [
    (dict(m=0), EINVAL), (dict(m=65), EUNSUP), (dict(m=65, hq=8), EUNSUP), (dict(q=0), EINVAL),
    (dict(q=FAKE + 2), EINVAL), (dict(out=0), EINVAL), (dict(k=-1), EINVAL), (dict(idx=0), EINVAL),
    (dict(scale=float("inf")), EINVAL), (dict(hq=12), EINVAL), (dict(k=8200), EUNSUP),
    (dict(d=dict(v_pool=0)), EINVAL),
])
def test_verify_attn_rejects(L, kw, code):
    d = desc(**kw.get("d", {}))
    r = L.kvsel_verify_attn(ctypes.byref(d), kw.get("q", FAKE), kw.get("m", 4), kw.get("hq", 16),
                            kw.get("scale", 0.088), kw.get("idx", FAKE), kw.get("k", 5), kw.get("out", FAKE), None,
                            None)
    assert r == code
    assert L.kvsel_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), EINVAL), (dict(k=0), EINVAL), (dict(v=0), EINVAL), (dict(cu=0), EINVAL), (dict(out=0), EINVAL),
    (dict(q=FAKE + 2), EINVAL), (dict(out=FAKE + 4), EINVAL), (dict(batch=0), EINVAL), (dict(hq=12), EINVAL),
    (dict(hkv=0), EINVAL), (dict(max_len=-1), EINVAL), (dict(scale=float("nan")), EINVAL), (dict(scale=-0.1), EINVAL),
    (dict(max_len=1 << 28, hq=64, hkv=8), EUNSUP),
])
def test_prefill_attn_rejects(L, kw, code):
    r = L.kvsel_prefill_attn(kw.get("q", FAKE), kw.get("k", FAKE), kw.get("v", FAKE), kw.get("cu", FAKE),
                             kw.get("batch", 1), kw.get("max_len", 100), kw.get("hq", 16), kw.get("hkv", 8),
                             kw.get("scale", 0.088), kw.get("out", FAKE), None, None)
    assert r == code
    assert L.kvsel_last_error()


def test_prefill_attn_empty_is_a_no_op(L):
    assert L.kvsel_prefill_attn(FAKE, FAKE, FAKE, FAKE, 1, 0, 16, 8, 0.088, FAKE, None, None) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), EINVAL), (dict(q=FAKE + 2), EINVAL), (dict(out=0), EINVAL), (dict(out=FAKE + 4), EINVAL),
    (dict(scale=0.0), EINVAL), (dict(rb=-1), EINVAL), (dict(rb=50, re=40), EINVAL), (dict(re=121), EINVAL),
    (dict(hq=12), EINVAL), (dict(d=dict(v_pool=0)), EINVAL), (dict(splits=0), EINVAL), (dict(splits=65), EINVAL),
    (dict(splits=2, lse=None), EINVAL), (dict(qps=0), EINVAL), (dict(logits=FAKE, ld=99), EINVAL),
    (dict(logits=FAKE, ld=100, qps=2), EINVAL), (dict(acc=2), EINVAL), (dict(acc=1, splits=2), EINVAL),
    (dict(acc=1, lse=None), EINVAL),
])
def test_shared_attn_rejects(L, kw, code):
    d = desc(shared_rows=120, **kw.get("d", {}))
    r = L.kvsel_shared_attn(ctypes.byref(d), kw.get("q", FAKE), kw.get("qps", 1), kw.get("hq", 16), kw.get("scale", 0.088),
                            kw.get("rb", 0), kw.get("re", 100), kw.get("splits", 1), kw.get("acc", 0), kw.get("out", FAKE),
                            kw.get("lse", FAKE), kw.get("logits", None), kw.get("ld", 0), None)
    assert r == code
    assert L.kvsel_last_error()


def test_shared_attn_block_limit(L):
    d = desc(shared_rows=20000, max_blocks_per_seq=1300, max_seq_len=20000, num_blocks=3000)
    assert L.kvsel_shared_attn(ctypes.byref(d), FAKE, 1, 16, 0.088, 0, 16385, 1, 0, FAKE, None, None, 0, None) == EUNSUP


@pytest.mark.parametrize("kw,code", [
    (dict(logits=0), EINVAL), (dict(idx=0), EINVAL), (dict(ld_logits=99), EINVAL), (dict(norm=1), EINVAL),
    (dict(k=0), EINVAL), (dict(scores=FAKE, ld=50), EINVAL), (dict(hq=12), EINVAL),
])
def test_select_logits_rejects(L, kw, code):
    d = desc()
    r = L.kvsel_select_logits(ctypes.byref(d), kw.get("logits", FAKE), kw.get("ld_logits", 100), kw.get("hq", 16),
                              0.088, kw.get("norm", 0), kw.get("k", 5), None, kw.get("idx", FAKE),
                              kw.get("scores", None), kw.get("ld", 0), None)
    assert r == code
    assert L.kvsel_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(o=0), EINVAL), (dict(lse=0), EINVAL), (dict(out=FAKE + 4), EINVAL), (dict(rows=-1), EINVAL),
    (dict(lse_out=0), EINVAL), (dict(parts=0), EINVAL), (dict(parts=65), EINVAL), (dict(o=FAKE + 8), EINVAL),
])
def test_merge_attn_rejects(L, kw, code):
    r = L.kvsel_merge_attn(kw.get("o", FAKE), kw.get("lse", FAKE), kw.get("parts", 2), kw.get("rows", 10),
                           kw.get("out", FAKE), kw.get("lse_out", FAKE), None)
    assert r == code


def test_merge_attn_empty_is_a_no_op(L):
    assert L.kvsel_merge_attn(FAKE, FAKE, 3, 0, FAKE, FAKE, None) == 0


def test_debug_status_of_the_release_and_debug_builds(L):
    """kvsel_debug_status: the release build holds no device checks (EUNSUPPORTED,
    outputs zeroed, no HIP call); the debug build registered every source
    file's check counters, so it reads them -- KVSEL_EHIP without a GPU, OK on
    one."""
    import ctypes
    import subprocess
    import sys
    n, c, d = ctypes.c_uint32(9), ctypes.c_uint32(9), ctypes.c_uint32(9)
    if os.environ.get("KVSEL_LIBRARY", "").endswith("libkvsel_debug.so"):
        pytest.skip("the debug build is loaded")
    assert L.kvsel_debug_status(ctypes.byref(n), ctypes.byref(c), ctypes.byref(d)) == EUNSUP
    assert (n.value, c.value, d.value) == (0, 0, 0)
    assert L.kvsel_debug_status(None, None, None) == EUNSUP
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    dbg = os.path.join(root, "decode_focal_layer_amd", "libkvsel_debug.so")
    if not os.path.exists(dbg):
        from decode_focal_layer_amd import build
        build.build(debug=True)
    probe = ("import ctypes; L = ctypes.CDLL(%r); L.kvsel_last_error.restype = ctypes.c_char_p; "
             "n = ctypes.c_uint32(9); print(L.kvsel_debug_status(ctypes.byref(n), None, None), n.value)" % dbg)
    r = subprocess.run([sys.executable, "-c", probe], capture_output=True, text=True, timeout=120)
    st, nv = (int(x) for x in r.stdout.split())
    assert st in (0, -4) and nv == 0, r.stdout + r.stderr
