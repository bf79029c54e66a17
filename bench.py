"""Benchmark of the block-causal paged attention hot path on one MI355X.

One step = the whole path over one batch of synthetic input: build_tile_mask (tile
classes, physical tile pages and the split-KV plan), attn_block_causal_paged, and
kv_commit_block of the active blocks. Inputs are resident in HBM before timing starts.
Before every timed step a 1 GiB buffer is overwritten so that neither L2 nor the 256 MB
Infinity Cache still holds the KV cache (one layer's cache is cold when that layer runs
again in a real decode step); a pair of HIP events on the stream the kernels run on
brackets each timed step. The per-call breakdown comes from as many further cold steps
with events between the calls (an event between two calls idles the GPU for a few
microseconds, so those steps are not timed as steps). A warm (no flush, back-to-back)
figure is reported beside it.

Prints one JSON line. `value` is microseconds per step (lower is better); `roofline`
rates the dominant kernel (attention) against MI355X's HBM or bf16 matrix peak on
algorithmic bytes/FLOPs; `cpu_baseline` is the CPU oracle timed on a bounded sample.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/decode-step + useful TFLOP/s & KV GB/s (% of MI355X roofline)"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2516.6     # 256 CU x 4096 dense bf16 FLOP/clk x 2.4 GHz
FP32_PEAK_TFLOPS = 157.3
# Which roof binds each workload (algorithmic FLOP/byte against the 314.6 FLOP/B ridge).
BOUND = {1: "hbm", 2: "hbm", 3: "mfma", 4: "mfma", 5: "hbm", 6: "hbm"}
# Sources whose code decides the attention call's memory traffic: the kernels, the planner
# that lays out their work, and the launch set-up.
KERNEL_SOURCES = ["attn_bf16.hip", "combine.hip", "tiles.hip", "abi.cpp"]
LAYERS = 32   # layers of the model step that is also timed as a captured graph


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", type=int, default=2, help="workload number 1-6 (default 2)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work to sample")
    p.add_argument("--calib-copy", action="store_true", help="also run a plain copy kernel of known size")
    p.add_argument("--no-graph", action="store_true", help="skip the captured 32-layer model step")
    p.add_argument("--window", type=int, default=0,
                   help="sliding window in positions (mode A workloads; 0 = none)")
    p.add_argument("--live-in-cache", action="store_true",
                   help="live keys/values already in the pool at kv_len + i: attention reads one "
                        "paged source and the commit moves only block ids")
    p.add_argument("--also", default="4,5,6,3",
                   help="comma-separated workloads whose attention call is also timed (cold, with its "
                        "own roofline) on the default line; '' for none")
    p.add_argument("--also-steps", type=int, default=20, help="timed calls per --also workload")
    p.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="no GPU: turn the counter_collection.csv files of two rocprofv3 --pmc runs "
                        "(FETCH_SIZE, then WRITE_SIZE) of `bench.py --calib-copy` into "
                        "profiles/attn_traffic_C<config>.json and .md")
    return p.parse_args()


CALIB_BYTES = 1 << 28        # the --calib-copy copy: 256 MiB read and 256 MiB written


def summarize_traffic(args):
    """HBM bytes per cold attention call from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by what the same counter reads for the 256 MiB calibration copy (an elementwise
    multiply by one, 256 MiB in and 256 MiB out)."""
    import csv
    import numpy as np

    def per_dispatch(path):
        rows = {}
        for r in csv.DictReader(open(path)):
            rows.setdefault(int(r["Dispatch_Id"]), [r["Kernel_Name"], 0.0])[1] += float(r["Counter_Value"])
        return [rows[k] for k in sorted(rows)]

    out = {}
    for name, path in (("fetch", args.summarize_traffic[0]), ("write", args.summarize_traffic[1])):
        d = per_dispatch(path)
        copies = [v for k, v in d if "MulFunctor" in k]
        calib = float(np.median(copies[-5:])) * 1024.0
        factor = CALIB_BYTES / calib
        calls, commits, cur = [], [], None
        for k, v in d:
            if "attn_bf16_kernel" in k or "attn_bf16_narrow_kernel" in k or "attn_f32_kernel" in k:
                cur = [v]
                calls.append(cur)
            elif "combine_kernel" in k and cur is not None:
                cur.append(v)
            elif "commit_kernel" in k:
                commits.append(v)
        cold = calls[args.warmup:args.warmup + args.steps]
        cold_commits = commits[args.warmup:args.warmup + args.steps]
        out[name] = {"calib_counter_bytes": calib, "factor": factor,
                     "bytes_per_call": float(np.median([sum(c) for c in cold])) * 1024.0 * factor,
                     "attn_kernel_bytes": float(np.median([c[0] for c in cold])) * 1024.0 * factor,
                     "commit_kernel_bytes": (float(np.median(cold_commits)) * 1024.0 * factor
                                             if cold_commits else None),
                     "cold_calls": len(cold)}
    rec = {"config": args.config, "kernel_hash": kernel_hash(),
           "hbm_bytes_per_call": out["fetch"]["bytes_per_call"] + out["write"]["bytes_per_call"],
           "fetch": out["fetch"], "write": out["write"],
           "commands": [f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o f -- python3 bench.py "
                        f"--config {args.config} --steps {args.steps} --warmup {args.warmup} --no-cpu-baseline --no-graph --calib-copy",
                        f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o w -- python3 bench.py "
                        f"--config {args.config} --steps {args.steps} --warmup {args.warmup} --no-cpu-baseline --no-graph --calib-copy",
                        f"python3 bench.py --config {args.config} --steps {args.steps} --warmup {args.warmup} "
                        f"--summarize-traffic <fetch csv> <write csv>"]}
    base = os.path.join(ROOT, "profiles", f"attn_traffic_C{args.config}")
    json.dump(rec, open(base + ".json", "w"), indent=1)
    case_name = f"C{args.config}"
    with open(base + ".md", "w") as f:
        f.write(f"# HBM traffic of one cold attention call, {case_name}\n\n")
        f.write("Counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch), two separate rocprofv3 --pmc runs,\n")
        f.write("each scaled by the same counter's reading for a 256 MiB device-to-device copy in the same run.\n\n")
        for c in rec["commands"]:
            f.write(f"    {c}\n")
        f.write("\n| counter | calib copy (counter bytes) | factor | per call, scaled (bytes) | attention kernel only |\n")
        f.write("|---|---|---|---|---|\n")
        for name in ("fetch", "write"):
            o = out[name]
            f.write(f"| {name.upper()}_SIZE | {o['calib_counter_bytes']:.4g} | {o['factor']:.4f} | "
                    f"{o['bytes_per_call']:.4g} | {o['attn_kernel_bytes']:.4g} |\n")
        f.write(f"\nHBM bytes per call (fetch + write): {rec['hbm_bytes_per_call']:.4g}; kernel code hash (comments stripped) "
                f"{rec['kernel_hash']} (bench.py reports it as roofline.traffic only while the hash matches).\n")
        if out["fetch"]["commit_kernel_bytes"] is not None:
            cf, cw = out["fetch"]["commit_kernel_bytes"], out["write"]["commit_kernel_bytes"]
            f.write(f"\nThe step's kv_commit_block (commit_kernel), same runs: {cf:.4g} bytes fetched and {cw:.4g} "
                    f"written per call ({cf + cw:.4g} in all).\n")
    print(json.dumps(rec))


def workload_stats(case, window=0):
    """Useful FLOPs (4*d per visible (row, key, query head)) and algorithmic bytes.

    With a sliding window W, live row i sees only keys fewer than W positions before it: in
    mode A committed row j sits at position j and live row i at kv_len + i, so live row i sees
    the committed rows j > kv_len + i - W and the live rows j > i - W of its block or earlier
    ones; in mode B the workload's positions decide. Only the committed rows that some live
    row sees count as bytes.
    """
    import numpy as np
    d, Hq, Hkv = case.head_dim, case.num_q_heads, case.num_kv_heads
    esize = 2 if case.dtype == "bf16" else 4
    visible = 0
    cached_rows = 0
    for s in range(case.batch):
        ql, kl = int(case.q_lens[s]), int(case.kv_len[s])
        if case.q_blk is None:
            i = np.arange(ql)
            live = np.minimum(ql, (i // case.block_size + 1) * case.block_size)
            if window:
                cached = np.clip(window - 1 - i, 0, kl)
                live = live - np.maximum(0, i - window + 1)
                visible += int((cached + live).sum())
                cached_rows += min(kl, window - 1)
            else:
                visible += int((kl + live).sum())
                cached_rows += kl
        elif window:
            # Mode B with a window: pairs with a block id not later and a position fewer than
            # W before the row's (positions of the multi-canvas layout).
            lo = int(case.cu_q[s])
            qb, qp = case.q_blk[lo:lo + ql].astype(np.int64), case.q_pos[lo:lo + ql].astype(np.int64)
            j = np.arange(kl)
            slots = case.page_table[s, j // case.page_size].astype(np.int64) * case.page_size + j % case.page_size
            kb = np.concatenate([case.kv_blk[slots].astype(np.int64), qb])
            kp = np.concatenate([case.kv_pos[slots].astype(np.int64), qp])
            vis = (kb[None, :] <= qb[:, None]) & (qp[:, None] - kp[None, :] < window)
            visible += int(vis.sum())
            cached_rows += int(vis[:, :kl].any(axis=0).sum())
        else:
            qb = np.sort(case.q_blk_seqs[s])
            kb = np.sort(case.kv_blk_seqs[s])
            rows = case.q_blk_seqs[s]
            visible += int(np.searchsorted(kb, rows, side="right").sum()
                           + np.searchsorted(qb, rows, side="right").sum())
            cached_rows += kl
    flops = 4.0 * d * Hq * visible
    cached_kv = float(cached_rows) * Hkv * d * esize * 2
    live_kv = float(case.total_q) * Hkv * d * esize * 2
    q_o = float(case.total_q) * Hq * d * esize * 2
    return flops, cached_kv, live_kv, q_o


def kernel_hash():
    """Hash of the attention kernels' code with comments and layout stripped, so that a
    change of comments alone does not mark the committed counter summaries stale."""
    h = hashlib.sha256()
    for n in KERNEL_SOURCES + ["bcp_internal.h"]:
        t = open(os.path.join(ROOT, "block_causal_paged_amd", "csrc", n)).read()
        t = re.sub(r"/\*.*?\*/", "", t, flags=re.S)
        t = re.sub(r"//[^\n]*", "", t)
        h.update(" ".join(t.split()).encode())
    return h.hexdigest()[:16]


def traffic_from_profile(cfg):
    """HBM bytes per attention call from the committed counter summary, or None when the
    kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"attn_traffic_C{cfg}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_hash") != kernel_hash():
        return None
    return rec.get("hbm_bytes_per_call")


def cpu_baseline(case, budget_s, window=0):
    """The oracle as it stands, over whole sequences of the same workload in order, pass
    after pass, until the budget is spent; scaled to microseconds per full step by the
    number of query rows covered. The BLAS pool is held to the cores this process may run
    on (its affinity mask), or to the pool's own size if that is smaller (the share a job
    is given), and `cores` reports that count."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle
    affinity = len(os.sched_getaffinity(0))
    pool = max([t.get("num_threads", 1) for t in threadpool_info()] + [1])
    threads = max(1, min(affinity, pool))
    with threadpool_limits(limits=threads):
        return _cpu_baseline_run(case, budget_s, window, threads, affinity, oracle, np)


def _cpu_baseline_run(case, budget_s, window, threads, affinity, oracle, np):
    t0 = time.perf_counter()
    rows_done = 0
    seqs = 0
    while True:
        s = seqs % case.batch
        oracle.attention_rows(case.q, case.k_new, case.v_new, case.k_cache, case.v_cache, case.cu_q,
                              case.kv_len, case.page_table, case.page_size, case.num_pages, s,
                              block_size=case.block_size, q_blk=case.q_blk, kv_blk=case.kv_blk,
                              window=window or None,
                              q_pos=case.q_pos if window and case.q_blk is not None else None,
                              kv_pos=case.kv_pos if window and case.q_blk is not None else None)
        rows_done += int(case.q_lens[s])
        seqs += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    steps = rows_done / max(1, case.total_q)
    per_step_us = dt / steps * 1e6
    what = (f"{seqs // case.batch} full passes over the {case.batch} sequences" + (f" and {seqs % case.batch} more"
            if seqs % case.batch else "")) if seqs >= case.batch else f"sequences 0..{seqs - 1} of {case.batch}"
    return {"value": per_step_us, "unit": "us/step", "cores": threads, "kind": "oracle",
            "affinity_cores": affinity,
            "sample": f"float64 NumPy oracle, all heads, on {what} ({steps:.3g} steps of query rows) "
                      f"in {dt:.1f} s on {threads} BLAS threads, scaled to one step"}


def roofline_of(case, cfg, attn_us_mean, window=0):
    """(roofline dict without traffic, useful flops, cached/live K/V bytes, Q+O bytes)."""
    flops, cached_kv, live_kv, q_o = workload_stats(case, window)
    algo_bytes = cached_kv + live_kv + q_o
    bound = BOUND[cfg]
    if bound == "hbm":
        achieved, peak, unit = algo_bytes / (attn_us_mean * 1e-6) / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        peak = MFMA_BF16_PEAK_TFLOPS if case.dtype == "bf16" else FP32_PEAK_TFLOPS
        achieved, unit = flops / (attn_us_mean * 1e-6) / 1e12, "TFLOP/s"
    G = case.num_q_heads // case.num_kv_heads
    narrow = case.dtype == "bf16" and 64 % G == 0 and case.max_q_len * G <= 64
    kern = "attn_f32_kernel" if case.dtype != "bf16" else ("attn_bf16_narrow_kernel" if narrow else "attn_bf16_kernel")
    roof = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "kernel": f"attn_block_causal_paged ({kern} + combine_kernel)",
            "algorithmic_bytes": algo_bytes, "useful_flops": flops, "launch_us_mean": round(attn_us_mean, 3)}
    return roof, flops, cached_kv, live_kv, q_o


def spin_up(flush, ms=500.0, work=None):
    """Keep the GPU busy for about `ms` milliseconds with fills of the flush buffer, each followed
    by `work()` if given, so that its clocks have left the idle state before a timed region. After
    a second of idling (building a workload on the host), the first ~40 ms of calls run up to
    20% slower without this (measured on C4 and C5)."""
    import torch

    t0 = time.perf_counter()
    k = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            flush.fill_(k & 0xFF)
            if work is not None:
                work()
            k += 1
        torch.cuda.synchronize()


def measure_attention_only(cfg, steps, flush):
    """Cold attention calls of workload `cfg` (flush outside the events), with the roofline of
    the mean: the figure every gated workload gets on the default line."""
    import numpy as np
    import torch

    import block_causal_paged_amd as bcp
    from workloads import CONFIG_NAMES, config
    from workloads.device import DeviceCase

    case = config(cfg)
    dc = DeviceCase(case)
    meta = bcp.StepMeta(**dc.meta_kwargs())
    plan = torch.empty(bcp.plan_size(meta), dtype=torch.uint8, device="cuda")
    ws = torch.empty(max(1, bcp.attn_workspace_size(meta)), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(dc.q)
    bcp.build_tile_mask(meta, plan=plan)

    def call():
        bcp.attn_block_causal_paged(meta, dc.q, dc.k_new, dc.v_new, dc.k_cache, dc.v_cache, out, plan=plan,
                                    workspace=ws)

    spin_up(flush, work=call)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for k in range(steps):
        flush.fill_(k & 0xFF)
        evs[k][0].record()
        call()
        evs[k][1].record()
    torch.cuda.synchronize()
    us = np.array([e[0].elapsed_time(e[1]) * 1e3 for e in evs])
    roof, flops, cached_kv, live_kv, _ = roofline_of(case, cfg, float(us.mean()))
    roof["traffic"] = traffic_from_profile(cfg)
    rec = {"workload": f"C{cfg} {CONFIG_NAMES[cfg]}",
           "attention_us": {"median": round(float(np.median(us)), 3), "mean": round(float(us.mean()), 3),
                            "p10": round(float(np.percentile(us, 10)), 3),
                            "p90": round(float(np.percentile(us, 90)), 3), "calls": steps},
           "useful_tflops": round(flops / (us.mean() * 1e-6) / 1e12, 2),
           "kv_gbps": round((cached_kv + live_kv) / (us.mean() * 1e-6) / 1e9, 1),
           "roofline": roof}
    del dc, plan, ws, out
    torch.cuda.empty_cache()
    return rec


def main():
    args = parse()
    if args.summarize_traffic:
        summarize_traffic(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by sequence or kv head with no collective; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import block_causal_paged_amd as bcp
    from workloads import CONFIG_NAMES, config
    from workloads.device import DeviceCase

    cfg = args.config
    case = config(cfg)
    dc = DeviceCase(case)
    torch.cuda.synchronize()
    if args.window and case.q_blk is not None and case.q_pos is None:
        print("--window in mode B needs a workload with positions (C4)", file=sys.stderr)
        sys.exit(2)
    meta = bcp.StepMeta(**dc.meta_kwargs(), window=args.window, live_in_cache=args.live_in_cache)
    plan = torch.empty(bcp.plan_size(meta), dtype=torch.uint8, device="cuda")
    nqt, nkt = bcp.num_q_tiles(meta), bcp.num_k_tiles(meta)
    tile_class = torch.empty((case.batch, nqt, nkt), dtype=torch.uint8, device="cuda")
    nct = -(-case.max_kv_len // 64)
    phys = torch.empty((case.batch, max(nct, 1), max(1, 64 // case.page_size)), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(1, bcp.attn_workspace_size(meta)), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(dc.q)
    k_cache, v_cache = dc.k_cache, dc.v_cache
    dst = dc.kv_len
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")

    k_live, v_live = (None, None) if args.live_in_cache else (dc.k_new, dc.v_new)
    if args.live_in_cache:
        # The producer's job, done once before timing: the live rows go to their slots
        # (logical rows kv_len + i), where every step then reads them.
        bcp.kv_commit_block(bcp.StepMeta(**dc.meta_kwargs()), dc.k_new, dc.v_new, dc.cu_q, dst, k_cache, v_cache,
                            case.total_q)

    def attn_call(m):
        bcp.attn_block_causal_paged(m, dc.q, k_live, v_live, k_cache, v_cache, out, plan=plan, workspace=ws)

    def commit_call(m):
        # In place only the block ids move (mode B); in mode A nothing is launched.
        bcp.kv_commit_block(m, k_live, v_live, dc.cu_q, dst, k_cache, v_cache, case.total_q,
                            src_blk=dc.q_blk if args.live_in_cache else None,
                            kv_blk_out=dc.kv_blk if args.live_in_cache else None, n_src=case.total_q)

    def step(evs=None):
        if evs: evs[0].record()
        bcp.build_tile_mask(meta, tile_class=tile_class, phys_page=phys if nct else None, plan=plan)
        if evs: evs[1].record()
        attn_call(meta)
        if evs: evs[2].record()
        commit_call(meta)
        if evs: evs[3].record()

    spin_up(flush)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: cold steps, each a flush (outside the events) and then the whole step
    # bracketed by one pair of events.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        flush.fill_(k & 0xFF)
        evs[k][0].record()
        step()
        evs[k][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_us = np.array([e[0].elapsed_time(e[1]) * 1e3 for e in evs])

    # Per-call breakdown, in as many further cold steps with events between the calls. Each
    # event between two calls leaves the GPU idle for a few microseconds at that boundary,
    # so these steps are not the step time; the attention call's own events give the
    # duration the roofline uses.
    evc = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        flush.fill_(k & 0xFF)
        step(evc[k])
    torch.cuda.synchronize()
    cls_us = np.array([e[0].elapsed_time(e[1]) * 1e3 for e in evc])
    attn_us = np.array([e[1].elapsed_time(e[2]) * 1e3 for e in evc])
    com_us = np.array([e[2].elapsed_time(e[3]) * 1e3 for e in evc])

    # Warm steps: back to back, no flush.
    warm_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    n_warm = max(args.steps, 20)
    warm_ev[0].record()
    for _ in range(n_warm):
        step()
    warm_ev[1].record()
    torch.cuda.synchronize()
    warm_step_us = warm_ev[0].elapsed_time(warm_ev[1]) * 1e3 / n_warm
    attn_warm = []
    for _ in range(n_warm):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        attn_call(meta)
        e[1].record()
        attn_warm.append(e)
    torch.cuda.synchronize()
    attn_warm_us = float(np.median([e[0].elapsed_time(e[1]) * 1e3 for e in attn_warm]))

    # A model step of LAYERS layers (the tile mask built once, then each layer's attention
    # call and KV commit; every layer reuses this workload's buffers, so it runs warm), issued
    # call by call and replayed as one captured step graph, on the same side stream.
    graph_rec = None
    if not args.no_graph:
        meta_u = bcp.StepMeta(**dc.meta_kwargs(), check=False, window=args.window, live_in_cache=args.live_in_cache)
        gs = torch.cuda.Stream()

        def model_step():
            bcp.build_tile_mask(meta_u, tile_class=tile_class, phys_page=phys if nct else None, plan=plan)
            for _ in range(LAYERS):
                attn_call(meta_u)
                commit_call(meta_u)

        n_rep = 5
        with torch.cuda.stream(gs):
            model_step()
            ge = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ge[0].record(gs)
            for _ in range(n_rep):
                model_step()
            ge[1].record(gs)
            gs.synchronize()
            eager_us = ge[0].elapsed_time(ge[1]) * 1e3 / n_rep
            bcp.graph_begin(gs)
            model_step()
            graph = bcp.graph_end(gs)
            graph.launch(gs)
            ge[0].record(gs)
            for _ in range(n_rep):
                graph.launch(gs)
            ge[1].record(gs)
            gs.synchronize()
            graph_us = ge[0].elapsed_time(ge[1]) * 1e3 / n_rep
            graph.close()
        graph_rec = {"layers": LAYERS, "eager_us": round(eager_us, 2), "graph_us": round(graph_us, 2),
                     "warm": True, "stream": "side stream, default priority"}

    if args.calib_copy:
        # A plain elementwise kernel (not the runtime's blit) that reads and writes 256 MiB.
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
        dst_buf = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1.0, out=dst_buf)
        torch.cuda.synchronize()

    a_med = float(np.median(attn_us))
    a_mean = float(np.mean(attn_us))
    roof, flops, cached_kv, live_kv, q_o = roofline_of(case, cfg, a_mean, args.window)
    algo_bytes = cached_kv + live_kv + q_o
    roof["traffic"] = None if args.window or args.live_in_cache else traffic_from_profile(cfg)

    rec = {
        "metric": METRIC,
        "value": round(float(np.mean(step_us)), 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(float(np.mean(step_us)) / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic (seeded; shapes and distributions of the named workload)",
        "config": {"workload": f"C{cfg} {CONFIG_NAMES[cfg]}", "batch": case.batch,
                   "q_heads": case.num_q_heads, "kv_heads": case.num_kv_heads, "head_dim": case.head_dim,
                   "total_q": case.total_q, "kv_len_mean": float(case.kv_len.mean()),
                   "kv_len_max": int(case.kv_len.max()), "page_size": case.page_size,
                   "block_size": case.block_size, "mode": case.mode,
                   **({"window": args.window} if args.window else {}),
                   **({"live_in_cache": True} if args.live_in_cache else {})},
        "roofline": roof,
        "attention_us": {"median": round(a_med, 3), "mean": round(a_mean, 3),
                         "p10": round(float(np.percentile(attn_us, 10)), 3),
                         "p90": round(float(np.percentile(attn_us, 90)), 3),
                         "warm_median": round(attn_warm_us, 3)},
        "useful_tflops": round(flops / (a_mean * 1e-6) / 1e12, 2),
        "kv_gbps": round((cached_kv + live_kv) / (a_mean * 1e-6) / 1e9, 1),
        "hbm_frac": round(algo_bytes / (a_mean * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "mfma_frac": round(flops / (a_mean * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "build_tile_mask_us": round(float(np.mean(cls_us)), 3),
        "kv_commit_us": round(float(np.mean(com_us)), 3),
        "kv_commit_gbps": None if args.live_in_cache else round(2 * live_kv / (float(np.mean(com_us)) * 1e-6) / 1e9, 1),
        "warm_step_us": round(warm_step_us, 3),
        "model_step_graph": graph_rec,
        "timed_wall_s_incl_flush": round(wall, 4),
        "device": torch.cuda.get_device_name(0),
        "cus": torch.cuda.get_device_properties(0).multi_processor_count,
    }
    also = [int(x) for x in args.also.split(",") if x.strip()] if not (args.window or args.live_in_cache) else []
    also = [c for c in also if c != cfg]
    if also:
        # The other gated workloads' attention calls, each cold and with its own roofline.
        del dc, ws, out, plan
        torch.cuda.empty_cache()
        rec["other_workloads"] = {f"C{c}": measure_attention_only(c, args.also_steps, flush) for c in also}
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(case, args.cpu_budget, args.window)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
