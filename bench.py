#!/usr/bin/env python3
"""Benchmark: single-token decode attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long]

One step is one complete call of the library for the whole batch (the split-K
partial kernel plus, when the plan splits the keys, the log-sum-exp combine),
with every input already resident in HBM. Prints ONE JSON line:

  value        algorithmic bytes per step / wall time per step, in GB/s, where the
               algorithmic bytes are the live K and V rows plus q and out (for the
               sparse workloads: the gathered rows, the selection, q and out)
  roofline     the partial kernel (the one that streams K and V): algorithmic bytes
               per launch / its mean duration from HIP events recorded on its own
               stream around each launch of a separate sampling loop after the
               timed region, against 8 TB/s; the whole call (partial kernel and
               merge) is timed the same way and reported beside it
  cpu_baseline the fp64 oracle timed on this host's cores over a bounded sample of
               the same workload
  all_configs  (default workload only) the same measurements for the other four
               configurations: dense tiny, dense GQA, dense large batch, sparse

Workloads are the seeded synthetic inputs of ``workloads.py``; the default is the
long-context dense GQA workload (B=4, Hq=64, Hkv=8, D=128, k_len = capacity =
131072), whose K and V (2 GiB) are far larger than the 256 MB Infinity Cache.
Smaller workloads are rotated over several copies of K and V so that each step
reads from HBM rather than from that cache.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode attention KV-read GB/s (fraction of HBM peak) and µs/step"
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_partial.json")


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


ATTENTION_SOURCES = ("kernels.hip", "device_common.h", "launch.h")
SELECT_SOURCES = ("select.hip", "select.h")


def kernel_source_hash(files=ATTENTION_SOURCES) -> str:
    """Hash of the kernel sources with comments and whitespace removed, so that
    stored counter readings stay valid across comment-only edits."""
    h = hashlib.sha256()
    for fn in files:
        with open(os.path.join(ROOT, "decode_attention_05_amd", "csrc", fn)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_from_counters(workload: str):
    """HBM bytes per partial-kernel launch from committed rocprofv3 counter runs,
    or None when they are missing or were taken on a different kernel source."""
    try:
        with open(COUNTERS_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload)
    files = SELECT_SOURCES if workload in ("select", "select_one") else ATTENTION_SOURCES
    if not entry or entry.get("kernel_source_hash") != kernel_source_hash(files):
        return None
    return entry.get("hbm_bytes_per_launch")


def per_wave_runs(plan, B, Hkv, G, Sq) -> bool:
    """Whether the length-balanced pass takes one run per wave: at least as many
    key streams (sequence, kv head, head tile) as the grid has waves. A stream
    holds the largest divisor of G whose heads times Sq fit 16 query rows."""
    heads = max(d for d in range(1, 16 // Sq + 1) if G % d == 0)
    return B * Hkv * (G // heads) >= plan.balanced_wgs * 4


def build_inputs(workload, W):
    if workload in W.RAGGED_CASES:
        case = W.RAGGED_CASES[workload]
        log(f"generating {workload} inputs (seed {case.seed})")
        if case.page_size:
            q, k, v, table, lens = W.paged_inputs(case)
            layout = (f"paged cache of {k.shape[0]} pages x {case.page_size} rows, "
                      f"block table [{case.B}, {case.max_pages}]")
        else:
            q, k, v, lens = W.ragged_inputs(case)
            table = None
            layout = f"contiguous cache, capacity {case.len_hi}"
        host = dict(q=q, k=k, v=v, sel=None, lens=lens, table=table)
        toks = f", {case.seq_q} causal query tokens per sequence" if case.seq_q > 1 else ""
        desc = (f"{case.name}: dense decode with one length per sequence, B={case.B} "
                f"Hq={case.Hq} Hkv={case.Hkv} D={case.D}{toks}, lengths {int(lens.min())}.."
                f"{int(lens.max())} (sum {int(lens.sum())}), {layout}")
        cfg = dict(batch=case.B, num_q_heads=case.Hq, num_kv_heads=case.Hkv, head_dim=case.D,
                   max_k_len=case.len_hi, total_k_len=int(lens.sum()), page_size=case.page_size,
                   seq_q=case.seq_q)
        return case, host, 2 * k.nbytes, desc, cfg, case.algorithmic_bytes()
    if workload in W.DENSE_CASES:
        case = W.DENSE_CASES[workload]
        log(f"generating {workload} inputs (seed {case.seed})")
        q, k, v = W.dense_inputs(case)
        host = dict(q=q, k=k, v=v, sel=None)
        kv_bytes_alloc = 2 * k.nbytes
        desc = (f"{case.name}: dense decode, B={case.B} Hq={case.Hq} Hkv={case.Hkv} D={case.D} "
                f"capacity={case.capacity} k_len={case.k_len}")
        cfg = dict(batch=case.B, num_q_heads=case.Hq, num_kv_heads=case.Hkv, head_dim=case.D,
                   capacity=case.capacity, k_len=case.k_len)
        return case, host, kv_bytes_alloc, desc, cfg, case.algorithmic_bytes()
    case = W.SPARSE_CASES[workload]
    log(f"generating {workload} inputs (seed {case.seed})")
    q, k, v, sel = W.sparse_inputs(case)
    host = dict(q=q, k=k, v=v, sel=sel)
    desc = (f"{case.name}: index-selected sparse decode, B={case.B} Hq={case.Hq} Hkv={case.Hkv} "
            f"D={case.D} rows={case.rows} topk={case.topk} valid={case.valid_counts()}")
    cfg = dict(batch=case.B, num_q_heads=case.Hq, num_kv_heads=case.Hkv, head_dim=case.D,
               rows=case.rows, topk=case.topk)
    return case, host, 2 * k.nbytes, desc, cfg, case.algorithmic_bytes()


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(args, case, host, algo_bytes, W, threads=None, seconds=None):
    """Time the fp64 oracle (as it stands) on this host over a bounded sample."""
    import numpy as np

    import oracle
    threads = threads or oracle.default_threads()
    seconds = args.cpu_seconds if seconds is None else seconds
    rows_total = case.B * case.Hq
    ragged = "lens" in host
    # About one second of all-core work per probe; grow the sample to ~10 s of wall.
    # Ragged batches sample every sequence equally (query row r is sequence r % B).
    n = min(rows_total, max(1, threads))
    if ragged:
        n = case.B * max(1, -(-n // case.B))
    t_probe = 0.0
    while True:
        rows = np.arange(n, dtype=np.int64) % rows_total
        t0 = time.perf_counter()
        if ragged:
            flat = (rows % case.B) * case.Hq + (rows // case.B) % case.Hq
            for b in range(case.B):
                heads = flat[flat // case.Hq == b] % case.Hq
                if host["table"] is not None:
                    rows_b = int(host["table"].shape[1]) * case.page_size
                    kb = oracle.unpage(host["k"], host["table"][b:b + 1], rows_b)
                    vb = oracle.unpage(host["v"], host["table"][b:b + 1], rows_b)
                else:
                    kb, vb = host["k"][b:b + 1], host["v"][b:b + 1]
                for t in range(case.seq_q):
                    seen = oracle.visible_keys(int(host["lens"][b]), case.seq_q, t, True)
                    if seen > 0:
                        oracle.dense(np.ascontiguousarray(host["q"][b:b + 1, :, t:t + 1]), kb, vb,
                                     case.scale, seen, rows=heads, threads=threads)
        elif host["sel"] is None:
            oracle.dense(host["q"], host["k"], host["v"], case.scale, case.k_len, rows=rows,
                         threads=threads)
        else:
            oracle.sparse(host["q"], host["k"], host["v"], host["sel"], case.scale, case.rows,
                          rows=rows, threads=threads)
        t_probe = time.perf_counter() - t0
        if t_probe >= seconds or n >= (1 << 24):
            break
        grow = max(2.0, min(8.0, seconds / max(t_probe, 1e-3)))
        n = int(n * grow)
        if ragged:
            n = case.B * -(-n // case.B)
    per_step = t_probe * rows_total / n
    return {
        "value": round(algo_bytes / per_step / 1e9, 4), "unit": "GB/s", "cores": threads,
        "kind": "oracle", "cpu_model": cpu_model(),
        "sample": (f"{n} query rows (b, h) of the {rows_total} in one step"
                   f"{' (rows repeated)' if n > rows_total else ''}, {t_probe:.2f} s wall on "
                   f"{threads} threads, scaled to a full step ({per_step * 1e3:.1f} ms/step)"),
        "s_per_step": round(per_step, 6),
    }


def calibration_copy(torch):
    """A plain 1 GiB device-to-device copy: its FETCH_SIZE / WRITE_SIZE counters
    give the scale from counted to actual HBM bytes in the same process."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log("calibration copy: 1073741824 bytes read, 1073741824 bytes written")
    del src, dst


def bench_selection(args, torch, np, da, W):
    """The on-device selection builder on the sparse workload's shapes ("select":
    the split builder, several workgroups per token with a workspace;
    "select_one": one workgroup per token), or split builder + sparse attention
    as one step ("sparse_built"): 4 tokens, 65408 scored index candidates, 1920
    chosen, a 128-slot window ring, width 2048."""
    case = W.SPARSE_CASES["sparse"]
    n_idx = case.rows - case.window
    k_idx = case.topk - case.window
    rng = np.random.Generator(np.random.PCG64(90))
    scores = rng.standard_normal((case.B, n_idx), dtype=np.float32)
    pos = np.array([70000 + 13 * b for b in range(case.B)], np.int32)
    dsc = torch.from_numpy(scores).cuda()
    dpos = torch.from_numpy(pos).cuda()
    dsel = torch.empty((case.B, case.topk), dtype=torch.int32, device="cuda")
    sel_bytes = scores.nbytes + pos.nbytes + case.B * case.topk * 4
    built = args.workload == "sparse_built"
    one_wg = args.workload == "select_one"
    sws_bytes = 0 if one_wg else da.decode_attn_select_workspace(case.B, n_idx, k_idx, case.window,
                                                                 case.topk)
    sws = torch.empty(sws_bytes, dtype=torch.uint8, device="cuda") if sws_bytes else None

    def build_sel():
        if one_wg:
            da.decode_attn_build_selection(dsc, dpos, dsel, n_idx, k_idx, case.window, n_idx)
        else:
            da.decode_attn_build_selection_ws(dsc, dpos, dsel, n_idx, k_idx, case.window, n_idx,
                                              sws)
    if built:
        log("generating sparse inputs (seed 5)")
        q, k, v, _ = W.sparse_inputs(case)
        dq, dk, dv = W.to_dev(q), W.to_dev(k), W.to_dev(v)
        out = torch.empty((case.B, case.Hq, 1, case.D), dtype=torch.bfloat16, device="cuda")
        plan = da.decode_attn_plan(case.B, case.Hq, case.Hkv, case.D, case.rows,
                                   topk_max=case.topk, kv_batch=1)
        ws = da.workspace_for(plan)
        algo_bytes = sel_bytes + case.algorithmic_bytes() - case.B * case.topk * 4
    else:
        algo_bytes = sel_bytes

    def step():
        build_sel()
        if built:
            da.decode_attn_sparse(plan, dq, dk, dv, dsel, case.topk, out, case.scale, case.rows, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    every = max(1, args.events_every)
    timed = list(range(0, args.steps, every))   # timed steps whose builder launch is bracketed
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in timed]
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in timed]
    t0 = time.perf_counter()
    for i in range(args.steps):
        if i % every == 0:
            ev_b[i // every].record(stream)
        build_sel()
        if i % every == 0:
            ev_a[i // every].record(stream)
        if built:
            da.decode_attn_sparse(plan, dq, dk, dv, dsel, case.topk, out, case.scale, case.rows, ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern_ms = np.array([ev_b[j].elapsed_time(ev_a[j]) for j in range(len(timed))])
    us = (t1 - t0) * 1e6 / args.steps
    kern_us = float(kern_ms.mean()) * 1e3
    log(f"{us:.1f} us/step, selection kernel mean {kern_us:.1f} us")
    graph_us = None
    if not args.no_graph:
        # 16 steps per replay, as the attention workloads replay one step per K/V
        # set: the figure is the in-graph cost of a step, not a replay's own launch
        per_replay = 16
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(per_replay):
                step()
        graph.replay()
        torch.cuda.synchronize()
        reps = max(1, args.steps // per_replay)
        g0 = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        torch.cuda.synchronize()
        graph_us = (time.perf_counter() - g0) * 1e6 / (reps * per_replay)
        log(f"graph replay: {graph_us:.1f} us/step ({per_replay} steps per replay)")
    if args.calibrate_copy:
        calibration_copy(torch)
    cpu = None
    if not args.no_cpu_baseline:
        from oracle.selection import build_selection
        t = time.perf_counter()
        build_selection(scores[:1], pos[:1], n_idx, k_idx, case.window, n_idx, case.topk)
        per_token = time.perf_counter() - t
        cpu = {"value": round(sel_bytes / (per_token * case.B) / 1e9, 6), "unit": "GB/s",
               "cores": 1, "kind": "oracle",
               "sample": f"selection of 1 of {case.B} tokens, {per_token:.2f} s, scaled to {case.B}"}
    value = algo_bytes / (us * 1e-6) / 1e9
    desc = (("selection builder, one workgroup per token" if one_wg else
             "selection builder, 16 workgroups per token and a merge") +
            (" + sparse attention" if built else "") +
            f": B={case.B} candidates={n_idx} k={k_idx} window={case.window} topk={case.topk}")
    print(json.dumps({
        "metric": METRIC, "value": round(value, 3), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(us / 1e3, 6),
        "us_per_step": round(us, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32" if not built else "bf16", "data": "synthetic",
        "config": {"workload": desc, "algorithmic_bytes_per_step": algo_bytes},
        "roofline": {"bound": "hbm", "achieved": round(sel_bytes / (kern_us * 1e-6) / 1e9, 3),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(sel_bytes / (kern_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 6),
                     "traffic": traffic_from_counters(args.workload if not built else "select"),
                     "kernel": "selection builder (all its kernels)",
                     "kernel_us_mean": round(kern_us, 3), "kernel_launches_timed": len(kern_ms),
                     "bytes_per_launch": sel_bytes},
        "cpu_baseline": cpu,
        "graph_us_per_step": None if graph_us is None else round(graph_us, 3),
    }), flush=True)


ALL_CONFIGS = ("tiny", "gqa", "batch", "sparse")   # reported beside the default workload


def run_workload(args, workload, torch, np, da, W, *, steps, warmup, graph, ceiling, cpu):
    """Time one workload: `steps` timed steps after `warmup`, then separate
    sampling loops for the kernel durations; returns the JSON line's fields."""
    case, host, kv_alloc, desc, cfg, algo_bytes = build_inputs(workload, W)
    sparse = host["sel"] is not None
    sets = 1 if kv_alloc >= 2 * MALL_BYTES else max(4, math.ceil(2 * MALL_BYTES / kv_alloc))
    log(f"copying to device ({sets} K/V set{'s' if sets > 1 else ''})")
    dq = W.to_dev(host["q"])
    dks = [W.to_dev(host["k"])]
    dvs = [W.to_dev(host["v"])]
    for _ in range(sets - 1):
        dks.append(dks[0].clone())
        dvs.append(dvs[0].clone())
    dsel = W.to_dev_i32(host["sel"]) if sparse else None
    ragged = "lens" in host
    paged = ragged and host["table"] is not None
    if ragged:
        dlens = W.to_dev_i32(host["lens"])
        dtable = W.to_dev_i32(host["table"]) if paged else None
    B, Hq, D = case.B, case.Hq, case.D
    out = torch.empty((B, Hq, getattr(case, "seq_q", 1), D), dtype=torch.bfloat16, device="cuda")
    if ragged:
        cap = case.len_hi
        if paged:
            plan = da.decode_attn_plan(B, Hq, case.Hkv, D, cap, cap, page_size=case.page_size,
                                       max_pages_per_seq=case.max_pages,
                                       num_pages=host["k"].shape[0], seq_q=case.seq_q,
                                       causal=True, force_splits=args.force_splits)
        else:
            plan = da.decode_attn_plan(B, Hq, case.Hkv, D, cap, cap, ragged=True,
                                       seq_q=case.seq_q, causal=True,
                                       force_splits=args.force_splits)
        splits = plan.balanced_wgs
    elif sparse:
        plan = da.decode_attn_plan(B, Hq, case.Hkv, D, case.rows, topk_max=case.topk,
                                   kv_batch=case.kv_batch, force_chunk=args.force_chunk)
        splits = -(-case.topk // plan.chunk)
    else:
        plan = da.decode_attn_plan(B, Hq, case.Hkv, D, case.capacity, case.k_len,
                                   force_splits=args.force_splits, force_chunk=args.force_chunk)
        splits = plan.num_splits_max
    ws = da.workspace_for(plan)

    append = args.with_append and not sparse and not ragged
    one_call = args.step and not sparse
    Sq = getattr(case, "seq_q", 1)
    if append or one_call:
        rng = np.random.Generator(np.random.PCG64(7))
        nshape = (B, case.Hkv, Sq if one_call else 1, D)
        kn = W.to_dev(W.f32_to_bf16_bits(rng.standard_normal(nshape, np.float32)))
        vn = W.to_dev(W.f32_to_bf16_bits(rng.standard_normal(nshape, np.float32)))
        algo_bytes += 2 * 2 * B * case.Hkv * nshape[2] * D * 2  # new rows read and written
    if append:
        pos_dev = torch.full((B,), case.k_len - 1, dtype=torch.int32, device="cuda")
    if one_call and not ragged:
        # fixed-length workloads: every sequence at k_len, through the length-balanced kernel
        plan = da.decode_attn_plan(B, Hq, case.Hkv, D, case.capacity, case.k_len, ragged=True)
        ws = da.workspace_for(plan)
        dlens = torch.full((B,), case.k_len, dtype=torch.int32, device="cuda")
        dtable = None
        splits = plan.balanced_wgs

    # Each K/V set's step, checked and marshalled once (PreparedCall): the timed
    # loop then only enqueues.
    def calls_for(kk, vv):
        if one_call:
            return [da.decode_attn_dense_step(plan, dq, kk, vv, kn, vn, dlens, out, case.scale,
                                              block_table=dtable if paged else None,
                                              workspace=ws, prepare=True)]
        if paged:
            return [da.decode_attn_dense_paged(plan, dq, kk, vv, dtable, dlens, out, case.scale,
                                               workspace=ws, prepare=True)]
        if ragged:
            return [da.decode_attn_dense_ragged(plan, dq, kk, vv, out, case.scale, dlens,
                                                workspace=ws, prepare=True)]
        if sparse:
            return [da.decode_attn_sparse(plan, dq, kk, vv, dsel, case.topk, out, case.scale,
                                          case.rows, ws, prepare=True)]
        seq = [da.decode_attn_append_kv(kk, vv, kn, vn, pos_dev, prepare=True)] if append else []
        return seq + [da.decode_attn_dense(plan, dq, kk, vv, out, case.scale, case.k_len, ws,
                                           prepare=True)]

    prepared = [calls_for(dks[i], dvs[i]) for i in range(sets)]

    def step(i):
        for call in prepared[i % sets]:
            call()

    # The measured streaming-read ceiling: a plain read of 4 GiB with the same
    # load style, timed with events on the current stream. It runs before the
    # warmup, so the timed steps also start from a GPU that has been busy.
    read_ceiling = None
    keep_alive = None
    if ceiling:
        buf = torch.ones(4 << 30, dtype=torch.uint8, device="cuda")
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        for _ in range(3):
            da.decode_attn_read_probe(buf, sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record()
        for _ in range(reps):
            da.decode_attn_read_probe(buf, sink)
        e1.record()
        torch.cuda.synchronize()
        read_ceiling = buf.numel() / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9
        log(f"streaming-read ceiling: {read_ceiling:.0f} GB/s")
        # Kept until the workload is done: memory handed back to the driver is
        # cleared in the background, which competes for HBM bandwidth (and the
        # graph capture below empties torch's cache).
        keep_alive = (buf, sink)

    log(f"{workload}: warmup {warmup} steps")
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    log(f"{workload}: timing {steps} steps")
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps

    # Kernel durations, in a sampling loop of their own after the timed region
    # (an event pair adds a few us to the step it brackets): the partial kernel
    # alone, with events the library records on its stream immediately around
    # that launch, then the whole call (partial kernel and merge) with events on
    # the same stream around the call.
    stream = torch.cuda.current_stream()
    n_samp = max(20, args.kernel_samples)
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(n_samp)]
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(n_samp)]
    for e in ev_b + ev_a:      # create the underlying hipEvent_t before handing it over
        e.record(stream)
    torch.cuda.synchronize()
    for j in range(n_samp):
        da.decode_attn_set_timing_events(ev_b[j].cuda_event, ev_a[j].cuda_event)
        step(j)
    da.decode_attn_set_timing_events(None, None)
    torch.cuda.synchronize()
    kern_ms = np.array([ev_b[j].elapsed_time(ev_a[j]) for j in range(n_samp)])
    for j in range(n_samp):
        ev_b[j].record(stream)
        step(j)
        ev_a[j].record(stream)
    torch.cuda.synchronize()
    call_ms = np.array([ev_b[j].elapsed_time(ev_a[j]) for j in range(n_samp)])

    # Warm: workloads rotated over several K/V copies (to defeat the 256 MB
    # Infinity Cache) are also timed on one copy, the cache-resident case.
    warm_us = None
    if sets > 1:
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        for i in range(steps):
            step(0)
        torch.cuda.synchronize()
        warm_us = (time.perf_counter() - w0) * 1e6 / steps
    value = algo_bytes / (ms_per_step * 1e-3) / 1e9
    kern_mean_s = float(kern_ms.mean()) * 1e-3
    call_mean_s = float(call_ms.mean()) * 1e-3
    achieved = algo_bytes / kern_mean_s / 1e9
    log(f"{workload}: {ms_per_step * 1e3:.1f} us/step, partial kernel mean {kern_mean_s * 1e6:.1f} us "
        f"(p10 {np.percentile(kern_ms, 10) * 1e3:.1f}, p90 {np.percentile(kern_ms, 90) * 1e3:.1f}), "
        f"whole call {call_mean_s * 1e6:.1f} us, {n_samp} launches sampled")

    # Plan-once decode: the same step captured once in a HIP graph (dense: the call
    # that reads k_len from device memory) and replayed; one replay runs every K/V
    # set once.
    graph_us = None
    if graph:
        klen_dev = torch.full((1,), 0 if (sparse or ragged) else case.k_len, dtype=torch.int32,
                              device="cuda")

        def gstep(i):
            # direct calls: they take torch's current stream, the capturing one
            kk, vv = dks[i % sets], dvs[i % sets]
            if ragged or one_call:
                for call in calls_for(kk, vv):  # prepared here, on the current stream
                    call()
            elif sparse:
                da.decode_attn_sparse(plan, dq, kk, vv, dsel, case.topk, out, case.scale, case.rows,
                                      ws)
            else:
                if append:
                    da.decode_attn_append_kv(kk, vv, kn, vn, pos_dev)
                da.decode_attn_dense_devlen(plan, dq, kk, vv, out, case.scale, klen_dev, ws)

        gstep(0)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(sets):
                gstep(i)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        reps = max(1, steps // sets)
        g0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        graph_us = (time.perf_counter() - g0) * 1e6 / (reps * sets)
        log(f"{workload}: graph replay: {graph_us:.1f} us/step")
        del g

    if args.calibrate_copy:
        calibration_copy(torch)

    traffic = traffic_from_counters(workload + ("+step" if one_call else ""))
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_step": round(ms_per_step * 1e3, 3),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": dict(workload=desc + (" (+ KV append per step)" if append else "")
                       + (" (one-call step: new rows written, then attended)" if one_call else ""),
                       splits=splits, kv_sets=sets,
                       algorithmic_bytes_per_step=algo_bytes, **cfg),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "measured_read_ceiling": None if read_ceiling is None else round(read_ceiling, 1),
            "frac_of_measured_ceiling": (None if read_ceiling is None
                                         else round(achieved / read_ceiling, 4)),
            "traffic": traffic,
            "kernel": (("attend_balanced_waves (length-balanced runs of one wave each)"
                        if per_wave_runs(plan, B, case.Hkv, Hq // case.Hkv, Sq)
                        else "attend_balanced (length-balanced stream of K and V)")
                       if ragged or one_call else "attend_partial (split-K stream of K and V)"),
            "kernel_us_mean": round(kern_mean_s * 1e6, 3),
            "kernel_us_median": round(float(np.median(kern_ms)) * 1e3, 3),
            "kernel_us_p10": round(float(np.percentile(kern_ms, 10)) * 1e3, 3),
            "kernel_us_p90": round(float(np.percentile(kern_ms, 90)) * 1e3, 3),
            "kernel_launches_timed": int(len(kern_ms)),
            "call_us_mean": round(call_mean_s * 1e6, 3),
            "call_frac": round(algo_bytes / call_mean_s / 1e9 / HBM_PEAK_GBS, 4),
            "bytes_per_launch": algo_bytes,
        },
        "cpu_baseline": None,
        "graph_us_per_step": None if graph_us is None else round(graph_us, 3),
        "warm_us_per_step": None if warm_us is None else round(warm_us, 3),
    }
    if cpu:
        log("timing the CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(args, case, host, algo_bytes, W)
        if workload in ("tiny", "sparse"):
            one = cpu_baseline(args, case, host, algo_bytes, W, threads=1,
                               seconds=args.cpu_seconds / 2)
            result["cpu_baseline"]["one_thread"] = {k: one[k] for k in ("value", "sample")}
    del prepared, dks, dvs, dq, out, ws, keep_alive
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return result


def config_summary(r):
    """The per-configuration record of all_configs."""
    rf = r["roofline"]
    return {
        "workload": r["config"]["workload"], "us_per_step": r["us_per_step"],
        "frac_of_hbm_peak": r["frac_of_hbm_peak"], "graph_us_per_step": r["graph_us_per_step"],
        "warm_us_per_step": r["warm_us_per_step"], "kernel_us_mean": rf["kernel_us_mean"],
        "kernel_frac": rf["frac"], "call_us_mean": rf["call_us_mean"],
        "call_frac": rf["call_frac"], "traffic": rf["traffic"],
        "algorithmic_bytes_per_step": r["config"]["algorithmic_bytes_per_step"],
        "splits": r["config"]["splits"], "kv_sets": r["config"]["kv_sets"],
        "steps": r["steps"], "kernel_launches_timed": rf["kernel_launches_timed"],
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="long",
                    choices=["tiny", "gqa", "long", "batch", "sparse", "sparse_mixed", "ragged",
                             "paged", "verify", "wide", "select", "select_one", "sparse_built"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-samples", type=int, default=50,
                    help="launches bracketed with HIP events after the timed region, for the "
                         "kernel durations (at least 20)")
    ap.add_argument("--events-every", type=int, default=8,
                    help="selection workloads: bracket the builder on every Nth timed step")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay timing of the plan-once call")
    ap.add_argument("--no-all-configs", action="store_true",
                    help="default workload only: skip the other four configurations")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--force-splits", type=int, default=0, help="dense split count (tuning)")
    ap.add_argument("--force-chunk", type=int, default=0,
                    help="keys (dense) or selection entries (sparse) per split (tuning)")
    ap.add_argument("--with-append", action="store_true",
                    help="dense: each step first appends the token's K/V rows at k_len - 1 "
                         "(a whole decode step: append, then attend)")
    ap.add_argument("--step", action="store_true",
                    help="dense: each step is one decode_attn_dense_step call, which writes the "
                         "pass's new K/V rows at the end of each prefix and attends (one kernel "
                         "pair instead of append + attention)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming-read ceiling measurement (a 4 GiB read probe)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after timing, run one plain 1 GiB device-to-device copy (a reference "
                         "dispatch of known traffic for hardware-counter runs)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported. Decode attention here shards with no exchange across (batch, kv head) "
              "units, so the whole-job figure for N GPUs is N times the one-GPU figure at a "
              "weak-scaled batch; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.step and args.workload in ("sparse", "sparse_mixed"):
        print("--step applies to the dense workloads", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import decode_attention_05_amd as da
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    da.library()

    if args.workload in ("select", "select_one", "sparse_built"):
        return bench_selection(args, torch, np, da, W)

    result = run_workload(args, args.workload, torch, np, da, W, steps=args.steps,
                          warmup=args.warmup, graph=not args.no_graph,
                          ceiling=not args.no_ceiling, cpu=not args.no_cpu_baseline)
    tuned = args.force_splits or args.force_chunk or args.with_append or args.step
    if args.workload == "long" and not args.no_all_configs and not tuned:
        # The other configurations: latency-bound ones get at least 200 timed steps.
        result["all_configs"] = {}
        for name in ALL_CONFIGS:
            r = run_workload(args, name, torch, np, da, W, steps=max(args.steps, 200),
                             warmup=max(args.warmup, 20), graph=not args.no_graph,
                             ceiling=False, cpu=False)
            result["all_configs"][name] = config_summary(r)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
