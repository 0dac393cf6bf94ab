"""Benchmark: FastOCR-style decode (28 layers, batch 32, 16 q / 8 kv heads,
6400 visual + 1024 text tokens, focal layers 3 and 14, top-320 per kv head,
warm-started top-k, 64-step cycle) through libkvsel on one MI355X.

A step is one decode step of all 28 layers over the batch: 2 focal layers
(dense attention fused with the focal scores, then top-k) and 26 layers of
gathered sparse attention (layers 0-2 reuse the previous step's deepest
focal set; at the first step of the cycle they attend densely).  Inputs (the
whole paged cache, every step's queries and sequence lengths) are resident
in HBM before timing starts.

Prints one JSON line.  --gpus N with N > 1 exits: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_c1_hbm_traffic.md")
KERNEL_SOURCES = ["decode_focal_layer_amd/csrc/attn.hip", "decode_focal_layer_amd/csrc/common.h",
                  "decode_focal_layer_amd/csrc/focal.h", "decode_focal_layer_amd/csrc/radix.h",
                  "decode_focal_layer_amd/csrc/kvsel_internal.h", "decode_focal_layer_amd/csrc/debug.h"]


def measured_traffic():
    """(HBM bytes per gathered-attention launch, those bytes / the algorithmic
    bytes of the launches counted) from the committed counter summary, if it
    was taken on the current kernel sources; else (None, None)."""
    import hashlib
    import re
    try:
        txt = open(TRAFFIC_FILE).read()
    except OSError:
        return None, None
    h = hashlib.sha256()
    for s in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, s), "rb").read())
    m = re.search(r"kernel-sources-sha256-16: ([0-9a-f]{16})", txt)
    t = re.search(r"Traffic per gathered-attention launch = [0-9.]+ \+ [0-9.]+ = ([0-9.]+) MB, ([0-9.]+) x", txt)
    if not m or not t or m.group(1) != h.hexdigest()[:16]:
        return None, None
    return float(t.group(1)) * 1e6, float(t.group(2))


def algorithmic_bytes(cfg, t: int, batch: int):
    """Bytes the method must move at step t of the cycle, per layer kind.

    K/V rows read once each (2 x 256 B per row per kv head), the query, the
    output, the focal scores (written by the scorer, read by top-k) and the
    kept indices (written by top-k, read by each sparse layer)."""
    hkv, hq, d = cfg.hkv, cfg.hq, cfg.head_dim
    n = cfg.prefix_len + t + 1
    row = 2 * d * 2                            # K + V bytes per row per kv head
    q_b = batch * hq * d * 2
    out_b = batch * hq * d * 4
    idx_b = batch * hkv * cfg.k * 4
    sc_b = batch * hkv * cfg.n_visual * 4
    dense = batch * hkv * n * row + q_b + out_b
    focal = dense + 2 * sc_b + idx_b           # scores written + read, indices written
    sparse = batch * hkv * (cfg.k + n - cfg.n_visual) * row + q_b + out_b + idx_b
    return dense, focal, sparse


def step_bytes(cfg, t, batch):
    dense, focal, sparse = algorithmic_bytes(cfg, t, batch)
    first = min(cfg.focal)
    n_focal = len(cfg.focal)
    n_pre = first
    n_sparse = cfg.layers - n_focal - (n_pre if t == 0 else 0)
    return n_focal * focal + (n_pre * dense if t == 0 else 0) + n_sparse * sparse


def cpu_baseline(w, cfg, t_sample: int, n_seq: int, cores_limit=None):
    """The oracle on the host cores for the same step, on n_seq of the batch's
    sequences (all 28 layers, every kv head): returns steps/s scaled to the
    whole batch.  cores_limit: BLAS threads (default: every core available)."""
    import torch
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import oracle as O

    cores = len(os.sched_getaffinity(0))
    G = cfg.group
    n = int(w.seq_len_np[t_sample, 0])
    # inputs for the sample, copied to host memory before timing
    kc = [w.k_pool[l][w.block_table[:n_seq].flatten().long()].cpu() for l in range(cfg.layers)]
    vc = [w.v_pool[l][w.block_table[:n_seq].flatten().long()].cpu() for l in range(cfg.layers)]
    mb = w.max_blocks
    local_table = np.arange(n_seq * mb).reshape(n_seq, mb)
    qc = w.q[t_sample].cpu()
    plan = O.focal_layer_plan(cfg.layers, cfg.focal, t_sample)
    with threadpool_limits(limits=cores_limit or cores):
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        t0 = time.perf_counter()
        for b in range(n_seq):
            for g in range(cfg.hkv):
                sets = {}
                # focal layers first: their sets feed the other layers; the layers before the
                # first focal layer take this step's deepest set in place of the previous
                # step's (same amount of work)
                for e in plan:
                    if e[0] != "focal":
                        continue
                    l = e[1]
                    K = O.logical_rows(kc[l], local_table[b], g, n)
                    V = O.logical_rows(vc[l], local_table[b], g, n)
                    qg = O.widen(qc[l, b, g * G:(g + 1) * G])
                    sets[l] = O.topk(O.focal_scores(qg, K, 0, cfg.n_visual, cfg.scale), cfg.k)
                    O.dense_attention(qg, K, V, cfg.scale)
                for e in plan:
                    if e[0] == "focal":
                        continue
                    l = e[1]
                    K = O.logical_rows(kc[l], local_table[b], g, n)
                    V = O.logical_rows(vc[l], local_table[b], g, n)
                    qg = O.widen(qc[l, b, g * G:(g + 1) * G])
                    if e[0] == "dense":
                        O.dense_attention(qg, K, V, cfg.scale)
                    else:
                        O.attention(qg, K, V, O.kept_rows(sets[e[3]], 0, cfg.n_visual, n), cfg.scale)
        dt = time.perf_counter() - t0
    steps_per_s = (n_seq / cfg.batch) / dt
    return {"value": steps_per_s, "unit": "steps/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"decode step t={t_sample} of the cycle, {n_seq} of {cfg.batch} sequences, all "
                      f"{cfg.layers} layers and {cfg.hkv} kv heads ({dt:.1f} s of host time), scaled to the "
                      f"full batch; {cores} host cores available"}


def oracle_parity(dec, w, cfg, n_seq: int):
    """The oracle leg's check of the benchmarked decoder itself: steps 0 and 1
    of the cycle on the GPU (the launch configuration timed above), then, for
    the first n_seq sequences, every kv head and all 28 layers of step 1
    against the oracle on the host.  Focal layers: the kept set by the tie-band
    rule (indices whose oracle score lies within 1e-6 of the k-th may differ)
    and the dense output; every other layer: its output against the oracle's
    attention over the rows the GPU's (validated) set keeps -- layers 0-2 the
    deepest focal layer's set of step 0, the others this step's set of the
    focal layer before them.  Tolerances: max abs 2e-3, relative L2 1e-3."""
    import torch
    from oracle import oracle as O

    last = max(cfg.focal)
    dec.step(0, w.q[0], w.seq_len[0])
    prev_set = dec.selection(last)[:n_seq].cpu().numpy()
    dec.step(1, w.q[1], w.seq_len[1])
    torch.cuda.synchronize()
    outs = dec.out[:, :n_seq].cpu().numpy()
    sets = {f: dec.selection(f)[:n_seq].cpu().numpy() for f in cfg.focal}
    n = int(w.seq_len_np[1, 0])
    G = cfg.group
    t0 = time.perf_counter()
    rows = w.block_table[:n_seq].flatten().long()
    table = np.arange(n_seq * w.max_blocks).reshape(n_seq, w.max_blocks)
    qc = w.q[1].cpu()
    worst_abs = worst_l2 = 0.0
    n_out = n_sets = exact = in_band = outside = 0
    for l, (kind, src) in enumerate(dec.plan(1)):
        kc, vc = w.k_pool[l][rows].cpu(), w.v_pool[l][rows].cpu()
        for b in range(n_seq):
            for g in range(cfg.hkv):
                K = O.logical_rows(kc, table[b], g, n)
                V = O.logical_rows(vc, table[b], g, n)
                qg = O.widen(qc[l, b, g * G:(g + 1) * G])
                if kind == "focal":
                    ref, _ = O.dense_attention(qg, K, V, cfg.scale)
                    sc = O.focal_scores(qg, K, 0, cfg.n_visual, cfg.scale)
                    gi = sets[l][b, g]
                    ok, nd = O.tie_band_check(gi, sc, cfg.k)
                    n_sets += 1
                    exact += int(ok and nd == 0)
                    in_band += int(ok and nd > 0)
                    outside += int(not ok)
                else:
                    which, ls = src
                    gi = prev_set[b, g] if which == "prev" else sets[ls][b, g]
                    ref, _ = O.attention(qg, K, V, O.kept_rows(gi, 0, cfg.n_visual, n), cfg.scale)
                got = outs[l, b, g * G:(g + 1) * G].astype(np.float64)
                worst_abs = max(worst_abs, float(np.abs(got - ref).max()))
                worst_l2 = max(worst_l2, float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)))
                n_out += 1
    ok = outside == 0 and worst_abs <= 2e-3 and worst_l2 <= 1e-3
    return {"ok": bool(ok), "sample": f"decode step t=1 of the cycle after t=0, sequences 0-{n_seq - 1}, all "
                                      f"{cfg.layers} layers and {cfg.hkv} kv heads",
            "outputs_checked": n_out, "max_abs_err": float(f"{worst_abs:.3e}"),
            "max_rel_l2": float(f"{worst_l2:.3e}"), "tolerance": {"max_abs": 2e-3, "rel_l2": 1e-3, "tie_band": 1e-6},
            "kept_sets_checked": n_sets, "kept_sets_exact": exact, "kept_sets_within_tie_band": in_band,
            "kept_sets_outside_tie_band": outside, "oracle_s": round(time.perf_counter() - t0, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--cpu-seqs", type=int, default=12, help="sequences in the oracle sample (0: skip)")
    ap.add_argument("--no-kernel-events", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain copy of this many MiB (counter calibration)")
    ap.add_argument("--deterministic", action="store_true",
                    help="attention with KVSEL_FLAG_DETERMINISTIC (rows summed in a fixed order)")
    ap.add_argument("--workload", default="c1", choices=["c0", "c1", "c2", "c3", "c4", "profile", "verify", "prefill"],
                    help="c1 (default) is the metric's workload; the others print their own line")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this hot path runs on one GPU; multi-GPU sharding is a design note only "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    from synth import gen
    from decode_focal_layer_amd import kvsel
    from decode_focal_layer_amd.decode import FocalDecoder

    kvsel.lib()
    dev = "cuda"
    if args.workload != "c1":
        return OTHER[args.workload](args)
    cfg = synth.C1
    t_gen = time.perf_counter()
    w = gen.make_focal(cfg, dev)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    print(f"[bench] generated C1 inputs in {t_gen:.1f} s "
          f"({sum(p.numel() for p in w.k_pool) * 4 / 1e9:.1f} GB of K/V)", file=sys.stderr, flush=True)
    max_len = int(w.seq_len_np.max())
    kvs = [kvsel.KV(w.k_pool[l], w.v_pool[l], w.block_table, w.seq_len[0], w.seg_begin, w.seg_end,
                    max_seq_len=max_len, max_seg_len=cfg.n_visual, min_seg_len=cfg.n_visual,
                    deterministic=args.deterministic)
           for l in range(cfg.layers)]
    dec = FocalDecoder(kvs, cfg.hq, cfg.k, cfg.focal, cfg.scale, cfg.n_visual, warm_start=True, device=dev)
    T = cfg.steps

    def run(i0, count, hook=None):
        for i in range(i0, i0 + count):
            t = i % T
            dec.step(t, w.q[t], w.seq_len[t], layer_hook=hook)

    run(0, args.warmup)
    torch.cuda.synchronize()

    # timed region: K steps, nothing else on the stream
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    run(args.warmup, args.steps)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop)
    ms_per_step = ms / args.steps
    steps_per_s = 1000.0 / ms_per_step
    total_bytes = sum(step_bytes(cfg, (args.warmup + i) % T, cfg.batch) for i in range(args.steps))
    gbs = total_bytes / (ms / 1e3) / 1e9

    # outside the timed region: one whole 64-step cycle (steps 0 .. 63, the
    # first of them with its dense layers), so that the rate over the cycle's
    # mean bytes is reported beside the rate over the timed steps' bytes
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for t in range(T):
        dec.step(t, w.q[t], w.seq_len[t])
    c1.record()
    torch.cuda.synchronize()
    cyc_ms = c0.elapsed_time(c1)
    cyc_bytes = sum(step_bytes(cfg, t, cfg.batch) for t in range(T))
    full_cycle = {"steps": T, "ms_per_step": round(cyc_ms / T, 4), "bytes_per_step_avg": int(cyc_bytes / T),
                  "hbm_gbs_algorithmic": round(cyc_bytes / (cyc_ms / 1e3) / 1e9, 1),
                  "hbm_frac_of_peak": round(cyc_bytes / (cyc_ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4)}

    # roofline of the dominant kernel (gathered sparse attention, 26 of 28 layers):
    # the same K steps again, with HIP events on the decode stream at the two ends
    # of every run of consecutive sparse layers (layers 4-13 and 15-27, plus 0-2
    # after the first step); a run's time / its launches = average launch time.
    roof = None
    if not args.no_kernel_events:
        marks = []          # (event_begin, event_end, launches, bytes)
        state = {}
        plans = {t: [e[0] for e in dec.plan(t)] for t in range(T)}

        def hook(l, kind, phase):
            t = state["t"]
            if phase == "begin" and kind == "sparse" and (l == 0 or plans[t][l - 1] != "sparse"):
                e = torch.cuda.Event(enable_timing=True)
                e.record()
                state["open"] = (e, 0, 0)
            if phase == "end" and kind == "sparse":
                e0, nl, nb = state["open"]
                nl += 1
                nb += algorithmic_bytes(cfg, t, cfg.batch)[2]
                state["open"] = (e0, nl, nb)
                nxt = plans[t][l + 1] if l + 1 < cfg.layers else None
                if nxt != "sparse":
                    e1 = torch.cuda.Event(enable_timing=True)
                    e1.record()
                    marks.append((e0, e1, nl, nb))

        torch.cuda.synchronize()
        for i in range(args.warmup, args.warmup + args.steps):
            t = i % T
            state["t"] = t
            dec.step(t, w.q[t], w.seq_len[t], layer_hook=hook)
        torch.cuda.synchronize()
        tot_ms = sum(a.elapsed_time(b) for a, b, _, _ in marks)
        launches = sum(n for _, _, n, _ in marks)
        nbytes = sum(nb for _, _, _, nb in marks)
        avg_us = tot_ms * 1e3 / launches
        bpl = nbytes / launches
        ach = bpl / (avg_us / 1e6) / 1e9
        traffic, traffic_ratio = measured_traffic()
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic,
                "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE x2.0 + WRITE_SIZE x1.0, calibrated "
                                "on a 1 GiB copy)",
                "traffic_over_algorithmic": traffic_ratio,
                "kernel": "attn_kernel<2,1024,4,0,true> (gathered sparse attention, streamed K/V)",
                "avg_launch_us": round(avg_us, 2), "bytes_per_launch": int(bpl), "launches_timed": launches}

    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    cpu = None
    if args.cpu_seqs > 0:
        cpu = cpu_baseline(w, cfg, 1, args.cpu_seqs)
        # the same oracle on one core, on a smaller sample of the same step
        one = cpu_baseline(w, cfg, 1, max(1, args.cpu_seqs // 3), cores_limit=1)
        cpu["single_core"] = {"value": one["value"], "unit": one["unit"], "cores": 1, "sample": one["sample"]}
        cpu["parity"] = oracle_parity(dec, w, cfg, min(4, args.cpu_seqs))

    line = {
        "metric": "decode attn steps/s (score + top-k + sparse attention, 28 layers)",
        "value": round(steps_per_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "c1_fastocr_decode: 28 layers, batch 32, 16q/8kv heads, head_dim 128, "
                               "6400 visual (80x80) + 1024 text tokens, focal layers {3,14}, top-320 per kv head, "
                               "64-step cycle, bf16 KV with fp32 accumulation",
                   "global_batch": cfg.batch, "seq_len": cfg.prefix_len, "parallelism": "single GPU",
                   "deterministic": bool(args.deterministic)},
        "tokens_per_s": round(steps_per_s * cfg.batch, 1),
        "hbm_gbs_algorithmic": round(gbs, 1),
        "hbm_frac_of_peak": round(gbs / PEAK_HBM_GBS, 4),
        "bytes_per_step_avg": int(total_bytes / args.steps),
        "full_cycle": full_cycle,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------------------
# the other workloads (parity cases of the test suite; timed here on request)
# ---------------------------------------------------------------------------

def _line(metric, value, unit, args, ms, workload, extra, higher=True):
    d = {"metric": metric, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": args.steps,
         "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": higher, "scaling": "weak",
         "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
         "config": {"workload": workload, "parallelism": "single GPU"}}
    d.update(extra)
    print(json.dumps(d), flush=True)


def _timed(fn, steps, warmup):
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(warmup, warmup + steps):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def bench_c0(args):
    """One decode step (fused focal pass + gathered attention) at the C0 shape;
    32 input copies rotate so repeats do not hit the last-level cache."""
    import torch
    import synth
    from synth import gen
    from decode_focal_layer_amd import kvsel
    cfg = synth.C0
    copies = []
    for c in range(32):
        w = gen.make_focal(synth.small(cfg, seed=cfg.seed + 1000 * c), "cuda")
        kv = kvsel.KV(w.k_pool[0], w.v_pool[0], w.block_table, w.seq_len[0], w.seg_begin, w.seg_end,
                      max_seq_len=cfg.prefix_len, max_seg_len=cfg.n_visual, min_seg_len=cfg.n_visual)
        copies.append((kv, w.q[0, 0].contiguous()))
    out = torch.empty((1, cfg.hq, 128), dtype=torch.float32, device="cuda")
    idx = torch.empty((1, cfg.hkv, cfg.k), dtype=torch.int32, device="cuda")
    ws = kvsel.Workspace("cuda")

    def step(i):
        kv, q = copies[i % len(copies)]
        kvsel.focal_attn(kv, q, cfg.hq, cfg.scale, out, cfg.k, idx, ws=ws)
        kvsel.gather_attn(kv, q, cfg.hq, cfg.scale, idx, cfg.k, out, ws=ws)

    ms = _timed(step, args.steps, args.warmup)
    dense = cfg.hkv * cfg.prefix_len * 512 + cfg.hq * 256 + cfg.hq * 512
    sparse = cfg.hkv * (cfg.k + cfg.n_always) * 512 + cfg.hq * 256 + cfg.hq * 512 + cfg.hkv * cfg.k * 4
    nbytes = dense + cfg.hkv * cfg.k * 4 + sparse
    _line("decode steps/s (focal pass + sparse attention, 1 layer)", 1000 / ms, "steps/s", args, ms,
          "c0_single_step: batch 1, 16q/8kv, 3584 visual + 512 text, top-179",
          {"bytes_per_step": nbytes, "hbm_gbs_algorithmic": round(nbytes / ms / 1e6, 1)})


def bench_profile(args):
    """Focal-layer profiling at the C1 shape: a warm-up step is the
    image-attention ratio of all 28 layers (batch 32, 16 heads, K only); the
    layer choice follows the last warm-up step."""
    import torch
    import synth
    from synth import gen
    from decode_focal_layer_amd import kvsel
    from decode_focal_layer_amd.decode import FocalProfiler
    cfg = synth.C1
    w = gen.make_focal(cfg, "cuda")
    max_len = int(w.seq_len_np.max())
    kvs = [kvsel.KV(w.k_pool[l], None, w.block_table, w.seq_len[0], w.seg_begin, w.seg_end,
                    max_seq_len=max_len, max_seg_len=cfg.n_visual, min_seg_len=cfg.n_visual)
           for l in range(cfg.layers)]
    W = 4
    prof = FocalProfiler(kvs, cfg.hq, cfg.scale, W, device="cuda")
    T = cfg.steps
    ms = _timed(lambda i: prof.step(i % W, w.q[i % T], w.seq_len[i % T]), args.steps, args.warmup)
    prof.pick(len(cfg.focal))   # first call loads the kernel
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(10):
        prof.pick(len(cfg.focal))
    b.record()
    torch.cuda.synchronize()
    pick_us = a.elapsed_time(b) * 1e3 / 10
    per_t = [cfg.layers * (cfg.batch * cfg.hkv * int(w.seq_len_np[t, 0]) * 256 + cfg.batch * cfg.hq * (256 + 4))
             for t in range(T)]
    nbytes = sum(per_t[(args.warmup + i) % T] for i in range(args.steps)) / args.steps
    _line("focal-layer profiling steps/s (image-attention ratio of 28 layers)", 1000 / ms, "steps/s", args, ms,
          "c1_profile: C1 cache (28 layers, batch 32, 16q/8kv, 6400 visual + 1024 text), ratio per layer "
          "from K only, top-2 layers after 4 warm-up steps",
          {"bytes_per_step_avg": int(nbytes), "hbm_gbs_algorithmic": round(nbytes / ms / 1e6, 1),
           "hbm_frac_of_peak": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4), "pick_us": round(pick_us, 2)})


def bench_c2(args):
    """One FastKV token-selective propagation (window scores on MFMA, pool,
    top-6554, gather of 6562 hidden rows); 6 input sets rotate."""
    import torch
    import synth
    from synth import gen
    from decode_focal_layer_amd import kvsel
    from decode_focal_layer_amd.fastkv import tsp_select
    cfg = synth.C2
    s0, s1 = cfg.seg
    sets = []
    for c in range(6):
        w = gen.make_window(synth.small(cfg, seed=cfg.seed + 1000 * c), "cuda")
        kv = kvsel.KV(w.k_pool, None, w.block_table, w.seq_len, w.seg_begin, w.seg_end,
                      max_seq_len=cfg.prompt, max_seg_len=s1 - s0, min_seg_len=s1 - s0)
        sets.append((kv, w.q, w.hidden))
    scores = torch.empty((1, 1, s1 - s0), dtype=torch.float32, device="cuda")
    idx = torch.empty((1, cfg.k), dtype=torch.int32, device="cuda")
    dst = torch.empty((cfg.k + cfg.window, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    ws = kvsel.Workspace("cuda")

    def step(i):
        kv, q, hid = sets[i % len(sets)]
        tsp_select(kv, q, cfg.hq, cfg.scale, cfg.k, cfg.pool, hidden=hid, window=cfg.window, scores=scores,
                   idx=idx, dst=dst, ws=ws)

    ms = _timed(step, args.steps, args.warmup)
    kbytes = cfg.prompt * cfg.hkv * 256
    nbytes = kbytes + cfg.window * cfg.hq * 256 + 2 * (s1 - s0) * 4 + 2 * cfg.k * 4 + \
        2 * (cfg.k + cfg.window) * cfg.hidden * 2
    flops = 2 * cfg.window * cfg.hq * cfg.prompt * 128
    _line("token selections/s (window score + pool + top-k + hidden gather)", 1000 / ms, "selections/s", args, ms,
          "c2_fastkv_tsp: prompt 32768, 32q/8kv, window 8, pool 7, top-6554 + 8 window rows, hidden 4096",
          {"bytes_per_selection": nbytes, "hbm_gbs_algorithmic": round(nbytes / ms / 1e6, 1),
           "mfma_gflop_per_selection": round(flops / 1e9, 3)})


def bench_c3(args):
    """FastKV decode under a 2048-row budget: decode steps of 32 layers (8
    aliased caches) after the one-off selection, which is timed separately."""
    import torch
    import synth
    from synth import gen
    from decode_focal_layer_amd import kvsel
    from decode_focal_layer_amd.fastkv import BudgetDecoder
    cfg = synth.C3
    s0, s1 = cfg.seg
    w = gen.make_budget(cfg, "cuda")
    kvs = [kvsel.KV(w.k_pool[p], w.v_pool[p], w.block_table, w.seq_len_sel, w.seg_begin, w.seg_end,
                    max_seq_len=cfg.src_len + cfg.steps, max_seg_len=s1 - s0, min_seg_len=s1 - s0)
           for p in range(cfg.phys_layers)]
    dec = BudgetDecoder(kvs, cfg.hq, cfg.k, cfg.layers, cfg.scale, cfg.window, cfg.pool, device="cuda")
    torch.cuda.synchronize()
    sel_ms = _timed(lambda i: dec.select(i % cfg.phys_layers, w.qwin[i % cfg.phys_layers], w.seq_len_sel),
                    cfg.phys_layers, 2)
    ms = _timed(lambda i: dec.step(w.q[i % cfg.steps], w.seq_len[i % cfg.steps]), args.steps, args.warmup)
    per_t = [cfg.layers * (cfg.batch * cfg.hkv * (cfg.k + cfg.recent + t + 1) * 512 + cfg.batch * cfg.hq * 768 +
                           cfg.batch * cfg.hkv * cfg.k * 4) for t in range(cfg.steps)]
    nbytes = sum(per_t[(args.warmup + i) % cfg.steps] for i in range(args.steps)) / args.steps
    sel_bytes = cfg.batch * cfg.hkv * cfg.src_len * 256
    _line("decode steps/s (gathered attention over a 2048-row budget, 32 layers)", 1000 / ms, "steps/s", args, ms,
          "c3_fastkv_budget_decode: batch 16, 32q/8kv, 131072-token context, 32 layers over 8 caches, "
          "2048 kept + 64 recent + generated rows",
          {"tokens_per_s": round(1000 / ms * cfg.batch, 1), "bytes_per_step_avg": int(nbytes),
           "hbm_gbs_algorithmic": round(nbytes / ms / 1e6, 1),
           "selection_ms_per_cache": round(sel_ms, 3), "selection_bytes_per_cache": sel_bytes,
           "selection_hbm_gbs_algorithmic": round(sel_bytes / sel_ms / 1e6, 1)})


def bench_c4(args):
    """HPD-style branched decode: 512 branches over one shared prefix, 28
    layers, focal layers {3, 14}, 32-step cycle."""
    import numpy as np
    import torch
    import synth
    from synth import gen
    from decode_focal_layer_amd import kvsel
    from decode_focal_layer_amd.decode import FocalDecoder
    cfg = synth.C4
    w = gen.make_focal(cfg, "cuda")
    max_len = int(w.seq_len_np.max())
    # the prefix rows are read by every branch: keep them cacheable
    kvs = [kvsel.KV(w.k_pool[l], w.v_pool[l], w.block_table, w.seq_len[0], w.seg_begin, w.seg_end,
                    max_seq_len=max_len, max_seg_len=cfg.n_visual, min_seg_len=cfg.n_visual,
                    shared_rows=cfg.prefix_len)
           for l in range(cfg.layers)]
    # sparse layers: the shared layout rows once per kv head for all branches, merged with each branch's own rows
    dec = FocalDecoder(kvs, cfg.hq, cfg.k, cfg.focal, cfg.scale, cfg.n_visual, device="cuda",
                       shared_tail=(cfg.n_visual, cfg.prefix_len))
    T = cfg.steps
    ms = _timed(lambda i: dec.step(i % T, w.q[i % T], w.seq_len[i % T]), args.steps, args.warmup)
    suf = w.suffix_len.astype(np.int64)
    logical, unique = [], []
    for t in range(T):
        tail = suf + t + 1
        n = cfg.prefix_len + tail
        lg = 2 * n.sum() + (cfg.layers - 2 - (3 if t == 0 else 0)) * (cfg.k + cfg.n_always + tail).sum() + \
            (3 * n.sum() if t == 0 else 0)
        un = cfg.layers * (cfg.prefix_len + tail.sum())      # every row once per layer at most
        logical.append(lg * cfg.hkv * 512)
        unique.append(un * cfg.hkv * 512)
    lb = sum(logical[(args.warmup + i) % T] for i in range(args.steps)) / args.steps
    ub = sum(unique[(args.warmup + i) % T] for i in range(args.steps)) / args.steps
    _line("branched decode steps/s (28 layers over 512 branches)", 1000 / ms, "steps/s", args, ms,
          "c4_hpd_branched: 512 branches, shared 3072 visual + 1024 layout prefix, suffix U[32,1024], "
          "16q/8kv, focal {3,14}, top-154",
          {"tokens_per_s": round(1000 / ms * cfg.batch, 1), "bytes_per_step_logical": int(lb),
           "bytes_per_step_unique_upper": int(ub),
           "hbm_gbs_logical": round(lb / ms / 1e6, 1)})


def bench_verify(args):
    """Draft verification at the C4 shape: every branch's m = 8 drafted
    tokens attend, in each of the 28 layers, over the kept visual rows (a
    fixed set of 154 per kv head), the 1024 layout rows, its suffix and,
    causally, the drafts (the last 8 rows of each branch)."""
    import numpy as np
    import torch
    import synth
    from synth import gen
    from decode_focal_layer_amd import kvsel
    cfg = synth.C4
    m = 8
    w = gen.make_focal(cfg, "cuda")
    seq = w.seq_len[cfg.steps - 1]
    n_np = w.seq_len_np[cfg.steps - 1].astype(np.int64)
    max_len = int(n_np.max())
    kvs = [kvsel.KV(w.k_pool[l], w.v_pool[l], w.block_table, seq, w.seg_begin, w.seg_end,
                    max_seq_len=max_len, max_seg_len=cfg.n_visual, min_seg_len=cfg.n_visual,
                    shared_rows=cfg.prefix_len)
           for l in range(cfg.layers)]
    g = torch.Generator(device="cuda").manual_seed(cfg.seed + 77)
    keys = torch.rand((cfg.batch * cfg.hkv, cfg.n_visual), generator=g, device="cuda")
    idx = keys.argsort(dim=1)[:, :cfg.k].sort(dim=1).values.to(torch.int32).view(cfg.batch, cfg.hkv, cfg.k)
    qs = [torch.randn((cfg.batch, m, cfg.hq, 128), generator=g, device="cuda").to(torch.bfloat16)
          for _ in range(4)]
    out = torch.empty((cfg.batch, m, cfg.hq, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((cfg.batch, m, cfg.hq), dtype=torch.float32, device="cuda")

    from decode_focal_layer_amd.decode import DraftVerifier
    # the shared layout rows once per kv head for every draft of every branch, merged with each branch's own rows
    vers = [DraftVerifier(kv, m, cfg.hq, cfg.scale, shared_tail=(cfg.n_visual, cfg.prefix_len)) for kv in kvs]

    def step(i):
        q = qs[i % len(qs)]
        for l in range(cfg.layers):
            vers[l].verify(q, idx, cfg.k, out, lse)

    ms = _timed(step, args.steps, args.warmup)
    rows = int((cfg.k + n_np - cfg.n_visual).sum())             # kept + layout + suffix (drafts included)
    per_layer = cfg.hkv * rows * 512 + cfg.batch * m * cfg.hq * (256 + 512 + 4) + cfg.batch * cfg.hkv * cfg.k * 4
    nbytes = cfg.layers * per_layer
    flops = cfg.layers * 4 * cfg.hkv * rows * (m * cfg.group) * 128
    _line("verification steps/s (8 drafts per branch, 28 layers over 512 branches)", 1000 / ms, "steps/s", args, ms,
          "c4_hpd_verify: 512 branches, shared 3072 visual + 1024 layout prefix, suffix U[32,1024] + 32, "
          "16q/8kv, 8 drafts, 154 kept visual rows per kv head",
          {"draft_tokens_per_s": round(1000 / ms * cfg.batch * m, 1), "bytes_per_step_logical": int(nbytes),
           "hbm_gbs_logical": round(nbytes / ms / 1e6, 1), "tflops": round(flops / ms / 1e9, 2)})


def bench_prefill(args):
    """TSP stage 2 at the C2 shape: one later layer's causal prefill over the
    6562 propagated tokens (6554 top-ranked + 8 window), 32q/8kv; 4 input
    sets rotate."""
    import torch
    import synth
    from decode_focal_layer_amd import kvsel
    cfg = synth.C2
    n, hq, hkv = cfg.k + cfg.window, cfg.hq, cfg.hkv
    g = torch.Generator(device="cuda").manual_seed(cfg.seed + 5)
    sets = [tuple(torch.randn((n, h, 128), generator=g, device="cuda").to(torch.bfloat16) for h in (hq, hkv, hkv))
            for _ in range(4)]
    cu = torch.tensor([0, n], dtype=torch.int32, device="cuda")
    out = torch.empty((n, hq, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((n, hq), dtype=torch.float32, device="cuda")

    def step(i):
        q, k, v = sets[i % len(sets)]
        kvsel.prefill_attn(q, k, v, cu, n, cfg.scale, out, lse)

    ms = _timed(step, args.steps, args.warmup)
    flops = 4 * 128 * hq * n * (n + 1) // 2          # S and P V over the causal triangle
    tfs = flops / ms / 1e9
    _line("TSP stage-2 prefill layers/s (causal attention over the propagated tokens)", 1000 / ms, "layers/s", args,
          ms, "c2_tsp_stage2: 6562 propagated tokens (6554 top-ranked + 8 window), 32q/8kv, head_dim 128",
          {"tflops": round(tfs, 1), "mfma_frac_of_bf16_peak": round(tfs / 2500.0, 4), "flop_per_layer": flops})


OTHER = {"c0": bench_c0, "c2": bench_c2, "c3": bench_c3, "c4": bench_c4, "profile": bench_profile,
         "verify": bench_verify, "prefill": bench_prefill}


if __name__ == "__main__":
    main()
