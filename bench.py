#!/usr/bin/env python3
"""Benchmark of the MoE dispatch -> combine hot path on one MI355X.

One step = the whole path on one batch: counts, padded prefix and stable
ranks, the bf16 scatter into the expert-contiguous, 128-row-padded buffer
(moe_dispatch_fused: layout and scatter in one call), then moe_combine
(weighted gather-sum + shared row).  Inputs are seeded synthetic tensors
already resident in HBM when the timed region starts.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps 100] [--warmup 10] [--workload skewed]
                    [--separate] [--eager]

`value` is algorithmic bytes per step (real rows only, never padding) divided
by the measured step time, in GB/s; `tokens_per_s` is tokens per step over the
same time.  The timed region holds the steps alone: no event is bound to a
launch inside it.  The `roofline` object covers the kernel that moves the most
bytes (combine): its algorithmic bytes per launch over its mean kernel time,
from HIP events bound to every launch (moe_time_next_launches: the runtime
stamps them with the kernel's own start and end on the launch stream) in
ROOFLINE_STEPS steps after the timed region; `kernels_ms` gives every
kernel's mean from the same steps.

The timed steps are replayed as captured HIP graphs of up to 20 steps each
(the largest count that divides --steps), the way a serving loop replays a
layer's launches; `--eager` launches every kernel from the host instead.
`--separate` runs layout and dispatch as two calls (moe_dispatch_layout,
moe_dispatch).  `cpu_baseline` times the CPU oracle on the same workload.
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
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X published HBM3E bandwidth
GRAPH_STEPS = 20        # most steps per captured graph (a pass of 20 MoE layers)
ROOFLINE_STEPS = 20     # steps after the timed region with every kernel launch timed
METRIC = "dispatch+combine achieved HBM GB/s and tokens/s, H=7168 E=256 K=8 bf16"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "combine_bf16_skewed_traffic.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "combine_moe_dispatch_layout_amd", "csrc", f)
                  for f in ("combine.hip", "moe_internal.h")]


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="skewed",
                   choices=["tiny", "decode", "skewed", "fp8", "large"])
    p.add_argument("--combine", default="bf16", choices=["bf16", "fp8"],
                   help="expert-output format read by the combine (fp8 = e4m3 + scales)")
    p.add_argument("--replicas", type=int, default=0,
                   help="split the N most popular experts into 4 replicas each and use the "
                        "replica-aware layout (probabilistic replica choice + count gathering; "
                        "moe_dispatch_fused_replicated, or with --separate the two calls)")
    p.add_argument("--ep", type=int, default=0,
                   help="rank-partitioned layout: experts split over N destination ranks, "
                        "moe_dispatch_layout_ep then moe_dispatch (separate calls)")
    p.add_argument("--sets", type=int, default=0,
                   help="buffer sets rotated across steps (0 = enough that no input stays "
                        "cache-resident between uses; see buffer_sets)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="CPU-oracle sample budget (0 disables the cpu_baseline leg)")
    p.add_argument("--separate", action="store_true",
                   help="layout and dispatch as two calls (moe_dispatch_layout or "
                        "moe_dispatch_layout_replicated, then moe_dispatch) instead of "
                        "moe_dispatch_fused or moe_dispatch_fused_replicated")
    p.add_argument("--fused", action="store_true",
                   help="layout + dispatch through moe_dispatch_fused (the default; one launch "
                        "for batches of at most 2048 pairs, else the layout launch reads the "
                        "token rows ahead for the scatter)")
    p.add_argument("--eager", action="store_true",
                   help="launch the timed steps' kernels from the host instead of replaying "
                        "captured HIP graphs")
    p.add_argument("--prepared", action="store_true",
                   help="with --eager: each call of a step made through a prepared call "
                        "(moe.prepare: arguments checked once per buffer set, then only "
                        "launched)")
    p.add_argument("--no-ceiling", action="store_true",
                   help="skip the practical-ceiling probe (streaming kernels with the "
                        "dispatch's and combine's read:write mixes)")
    p.add_argument("--copy-probe", action="store_true",
                   help="run only a plain 1 GiB device copy (counter calibration)")
    p.add_argument("--latency-floor", action="store_true",
                   help="print only per-launch times, in 10-launch HIP graphs, of an empty "
                        "kernel, the plain gather and scatter probes at the workload's layout "
                        "rows, and the path's own kernels (decode-sized latency floor)")
    p.add_argument("--layout-sweep", action="store_true",
                   help="print only moe_dispatch_layout kernel times at 32K to 64M pairs "
                        "(E = 256, K = 8), each launch timed by bound events")
    return p.parse_args()


# ---------------------------------------------------------------- byte model

def algorithmic_bytes(bs, h, e, k, shared=True, fp8=False, fp8_combine=False):
    """Bytes each kernel must move: real rows only, metadata once per kernel."""
    layout = 4 * bs * k + 4 * bs * k + 4 * e + 4 * (e + 1)
    if fp8:
        dispatch = 2 * bs * h + bs * k * (h + 4 * (h // 128)) + 8 * bs * k + 4 * (e + 1)
    else:
        dispatch = 2 * bs * h + 2 * bs * k * h + 8 * bs * k + 4 * (e + 1)
    rows_in = bs * k * (h + 4 * (h // 128)) if fp8_combine else 2 * bs * k * h
    combine = rows_in + (2 * bs * h if shared else 0) + 2 * bs * h + 12 * bs * k + 4 * (e + 1)
    return {"layout": layout, "dispatch": dispatch, "combine": combine}


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload):
    """HBM bytes per combine launch from the committed counter summary, or
    None when it is missing or the kernel source changed since."""
    if workload != "skewed" or not os.path.exists(TRAFFIC_FILE):
        return None
    txt = open(TRAFFIC_FILE).read()
    m_hash = re.search(r"^source_hash:\s*(\w+)", txt, re.M)
    m_bytes = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt, re.M)
    if not m_hash or not m_bytes or m_hash.group(1) != source_hash(KERNEL_SOURCES):
        return None
    return float(m_bytes.group(1))


# ---------------------------------------------------------------- CPU baseline

def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None where absent)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, budget_s, threads=1):
    """The oracle as it stands (plain C loops, gcc -O2), timed on this host
    over whole passes of the workload until the budget is spent.  With
    threads > 1 the layout stays one serial call and the dispatch and combine
    calls run on `threads` contiguous token slices at once (the C calls
    release the interpreter lock; the slices write disjoint rows)."""
    import concurrent.futures
    import numpy as np
    import oracle
    import workloads

    cap = oracle.capacity(w.bs, w.topk, w.experts, w.align)
    inp = workloads.make(w, rows_y=cap)
    ids, sc = inp["expert_ids"], inp["expert_scales"]
    x = workloads.bits(inp["x"])
    sh = None if inp["shared"] is None else workloads.bits(inp["shared"])
    out = np.full((cap, w.hidden), oracle.SENTINEL_BF16, np.uint16)  # pages touched up front
    y = out if w.identity_experts else workloads.bits(inp["y"])  # identity experts: y = dispatched rows
    k = w.topk
    cuts = [w.bs * i // threads for i in range(threads + 1)]
    pool = concurrent.futures.ThreadPoolExecutor(threads) if threads > 1 else None

    def token_slices(fn):
        if pool is None:
            fn(0, w.bs)
        else:
            list(pool.map(lambda i: fn(cuts[i], cuts[i + 1]), range(threads)))

    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        c, s, r, _ = oracle.layout(ids, w.experts, w.align)
        token_slices(lambda a, b: oracle.dispatch_bf16(x[a:b], ids[a:b], r[a * k:b * k], s,
                                                       w.experts, cap, out=out))
        token_slices(lambda a, b: oracle.combine(y, ids[a:b], r[a * k:b * k], s, sc[a:b],
                                                 None if sh is None else sh[a:b], w.experts))
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start >= budget_s and len(times) >= 2:
            break
    if pool is not None:
        pool.shutdown()
    t = sorted(times)[len(times) // 2]
    b = sum(algorithmic_bytes(w.bs, w.hidden, w.experts, w.topk, sh is not None).values())
    how = "single thread" if threads == 1 else (
        f"{threads} threads over token slices (layout serial)")
    return {"value": round(b / t / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "tokens_per_s": round(w.bs / t, 1),
            "ms_per_pass": round(t * 1e3, 2),
            "sample": f"whole {w.name} batch ({w.bs} tokens: layout + bf16 dispatch + "
                      f"combine), {len(times)} passes in {time.perf_counter() - t_start:.1f} s, "
                      f"median pass, {how}"}


# ---------------------------------------------------------------- GPU run

def copy_probe():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 5}), flush=True)


MALL_BYTES = 256 << 20      # MI355X Infinity Cache
SET_MEMORY_CAP = 48 << 30   # device memory the rotated buffer sets may take


def buffer_sets(w, cap, step_bytes, fp8_combine):
    """Buffer sets rotated across steps so that no input is served from a
    cache between its uses.  The streaming kernels read expert rows and the
    shared row with non-temporal loads and write with non-temporal stores,
    which do not allocate in the 256 MB Infinity Cache; the token rows x are
    read with ordinary loads and would stay resident across steps if few
    sets cycled.  So: enough sets that the other sets' x (the allocating
    traffic between two reads of one set's x) is at least twice the
    Infinity Cache, and a whole cycle moves at least 2 GiB; capped by
    SET_MEMORY_CAP of buffers and 64 sets.  At decode size the cap binds (each set holds
    full-capacity expert buffers for 1.8 MB of token rows), as its note in
    the output says."""
    x_bytes = 2 * w.bs * w.hidden
    per_set = (x_bytes * 3                                     # x, shared, out
               + cap * w.hidden * (1 if w.fp8 else 2)          # expand_x
               + cap * w.hidden * (1 if fp8_combine else 2))   # y (codes)
    by_cache = 1 + -(-2 * MALL_BYTES // x_bytes)
    by_volume = -(-(2 << 30) // step_bytes)
    return max(1, min(max(by_cache, by_volume), SET_MEMORY_CAP // per_set, 64))


def steps_per_graph(steps: int) -> int:
    """Steps per captured graph: the largest count up to GRAPH_STEPS that
    divides the timed steps, so that the timed region replays whole graphs."""
    return max(d for d in range(1, GRAPH_STEPS + 1) if steps % d == 0)


def per_launch_in_graphs(fn, launches=10, replays=30):
    """Median microseconds per launch of `fn` captured `launches` times in one
    HIP graph, each replay bracketed by events on the stream (the graph's
    launch gap included, as in a serving loop that replays a whole pass)."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(launches):
            fn()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(replays)]
    for a, z in evs:
        a.record()
        g.replay()
        z.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(z) for a, z in evs)
    return round(t[len(t) // 2] * 1e3 / launches, 2)


def latency_floor(moe, w, b, ids, scales, n_phys, cap, front, combine):
    """The decode-sized step against the latency floor of its launches: an
    empty kernel (one workgroup, and the combine's grid), the plain gather
    probe with the combine's reads at this routing's layout rows (K expert
    rows + the shared row per token, one row written: one dependent load of
    the row indices, then the rows), the scatter probe with the dispatch's
    writes at the same rows, and the path's own kernels, all in 10-launch
    graphs on one buffer set."""
    import torch
    lay = front(b)
    torch.cuda.synchronize()
    slots = (lay.ep_send_counts[ids.reshape(-1).long()].long()
             + lay.expand_idx.long()).view(w.bs, w.topk).to(torch.int32)
    cols = w.hidden // 2                          # int32 columns of a bf16 row
    grid_combine = w.bs * (-(-(w.hidden // 8) // 128))
    y_rows = torch.zeros((cap + w.bs, cols), dtype=torch.int32, device="cuda")
    out_rows = torch.empty((max(cap, w.bs), cols), dtype=torch.int32, device="cuda")
    shared_rows = (cap + torch.arange(w.bs, dtype=torch.int32, device="cuda"))[:, None]
    gather_src = torch.cat([slots, shared_rows], dim=1).reshape(-1).contiguous()
    scatter_dst = slots.reshape(-1).contiguous()
    x_rows = torch.zeros((w.bs, cols), dtype=torch.int32, device="cuda")
    res = {
        "empty_kernel_1_workgroup": per_launch_in_graphs(lambda: moe.moe_probe_empty(1)),
        f"empty_kernel_{grid_combine}_workgroups": per_launch_in_graphs(
            lambda: moe.moe_probe_empty(grid_combine)),
        "gather_probe_combine_reads": per_launch_in_graphs(
            lambda: moe.moe_probe_stream_mix(y_rows, out_rows, w.bs, w.topk + 1, 1,
                                             gather_src, None)),
        "scatter_probe_dispatch_writes": per_launch_in_graphs(
            lambda: moe.moe_probe_stream_mix(x_rows, out_rows, w.bs, 1, w.topk, None,
                                             scatter_dst)),
        "layout+dispatch": per_launch_in_graphs(lambda: front(b)),
        "combine": per_launch_in_graphs(lambda: combine(b, lay)),
        "step": per_launch_in_graphs(lambda: combine(b, front(b))),
    }
    return res


def layout_sweep(moe):
    """moe_dispatch_layout kernel time (all of its launches, each timed by
    events bound to it; median of 20 calls) at growing pair counts, E = 256,
    K = 8, routing (h_t + j) mod E with a seeded uniform h_t."""
    import numpy as np
    import torch
    out = {}
    for pairs in (1 << 15, 1 << 20, 1 << 22, 1 << 24, 1 << 26):
        bs, k, e = pairs // 8, 8, 256
        h = torch.from_numpy(np.random.default_rng(pairs).integers(0, e, bs, dtype=np.int32))
        ids = ((h[:, None] + torch.arange(k, dtype=torch.int32)) % e).to(torch.int32).cuda()
        lay = moe.moe_dispatch_layout(ids, e, 128)
        ws = torch.zeros(max(moe.moe_dispatch_layout_workspace_size(bs, k, e), 16),
                         dtype=torch.uint8, device="cuda")
        times = []
        for _ in range(23):
            pairs_ev = [(torch.cuda.Event(enable_timing=True),
                         torch.cuda.Event(enable_timing=True)) for _ in range(2)]
            for a, z in pairs_ev:
                a.record()
                z.record()
            moe.moe_time_next_launches(pairs_ev)
            moe.moe_dispatch_layout(ids, e, 128, out=lay, workspace=ws)
            used = 2 - moe.moe_time_unused_launches()
            moe.moe_time_next_launches([])
            torch.cuda.synchronize()
            times.append(sum(a.elapsed_time(z) for a, z in pairs_ev[:used]) * 1e3)
        times = sorted(times[3:])
        out[str(pairs)] = {"us": round(times[len(times) // 2], 2),
                           "ns_per_1k_pairs": round(times[len(times) // 2] * 1e3 / (pairs / 1e3),
                                                    3),
                           "launches": used}
        del ids, lay, ws
        torch.cuda.empty_cache()
    return out


def practical_ceiling(moe, w, slots, cap, out_row_bytes, launches=16):
    """GB/s of the plain streaming probe with the dispatch's 1 : K and the
    combine's (K + 1) : 1 row mixes at this workload's bf16 row size and
    token count, and of the scatter's writes alone (`scatter_writes`: K rows
    of `out_row_bytes` per token, the row read being one cache-resident row,
    write bytes counted), with the expert-side rows
      - in order (`in_order`),
      - randomly permuted (`random_rows`; seeded), and
      - at the real layout's slots of this routing (`layout_rows`: tokens in
        order, each token's K rows where the layout puts them),
    the token-side rows (x, shared, output) in order.  `slots` is the int64
    [BS, K] device tensor of the layout's rows.  Mean kernel time of
    `launches` launches (at most 16), each timed by HIP events bound to it,
    after 3 warm-up launches."""
    import numpy as np
    import torch
    bs, k, row_bytes = w.bs, w.topk, 2 * w.hidden
    cols = row_bytes // 4
    g = np.random.default_rng(12345)
    rows_y = max(bs * k, cap)
    layout_rows = slots.to(torch.int32).contiguous()
    out = {}
    one_row = torch.zeros(bs, dtype=torch.int32, device="cuda")
    for name, reads, writes in (("dispatch_mix", 1, k), ("combine_mix", k + 1, 1),
                                ("scatter_writes", 1, k)):
        mix_cols = out_row_bytes // 4 if name == "scatter_writes" else cols
        src_n = 1 if name == "scatter_writes" else (bs if writes > 1 else rows_y + bs)
        src = torch.zeros((src_n, mix_cols), dtype=torch.int32, device="cuda")
        dst = torch.empty((rows_y if writes > 1 else bs, mix_cols), dtype=torch.int32,
                          device="cuda")
        perm = torch.from_numpy(g.permutation(bs * k).astype(np.int32)).cuda().view(bs, k)
        shared_rows = (rows_y + torch.arange(bs, dtype=torch.int32, device="cuda"))[:, None]
        res = {}
        for order, expert_rows in (("in_order", None), ("random_rows", perm),
                                   ("layout_rows", layout_rows)):
            if name == "scatter_writes":  # one cached source row, K rows written
                src_rows = one_row
                dst_rows = None if expert_rows is None else expert_rows.reshape(-1).contiguous()
            elif expert_rows is None:   # contiguous: item i's rows i*R .. i*R+R-1
                src_rows = dst_rows = None
            elif writes > 1:          # dispatch: token row t, K copies to the expert rows
                src_rows, dst_rows = None, expert_rows.reshape(-1).contiguous()
            else:                     # combine: K expert rows, then the token's shared row
                src_rows = torch.cat([expert_rows, shared_rows], dim=1).reshape(-1).contiguous()
                dst_rows = None
            run = lambda: moe.moe_probe_stream_mix(src, dst, bs, reads, writes, src_rows,
                                                   dst_rows)
            for _ in range(3):
                run()
            pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                     for _ in range(launches)]
            for a, z in pairs:
                a.record()
                z.record()
            moe.moe_time_next_launches(pairs)
            for _ in range(launches):
                run()
            torch.cuda.synchronize()
            secs = sum(a.elapsed_time(z) for a, z in pairs) / 1e3 / launches
            moved = (bs * writes * out_row_bytes if name == "scatter_writes"
                     else bs * (reads + writes) * row_bytes)
            res[order] = round(moved / secs / 1e9, 1)
        out[name] = res
        del src, dst
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(the path is single-device; no collectives are built)", file=sys.stderr)
        sys.exit(2)
    if args.fused and args.separate:
        print("--fused and --separate exclude each other", file=sys.stderr)
        sys.exit(2)
    if args.ep and (args.replicas > 0 or args.fused):
        print("--ep runs the separate calls and takes no --replicas or --fused",
              file=sys.stderr)
        sys.exit(2)
    if args.prepared and not args.eager:
        print("--prepared launches from the host: it needs --eager", file=sys.stderr)
        sys.exit(2)
    if args.ep:
        args.separate = True
    # moe_dispatch_fused (moe_dispatch_fused_replicated with --replicas) is the
    # step's layout + dispatch unless asked otherwise.
    args.fused = not args.separate
    import torch
    if args.copy_probe:
        copy_probe()
        return

    import combine_moe_dispatch_layout_amd as moe
    import workloads

    moe.load_library()
    if args.layout_sweep:
        torch.cuda.set_device(0)
        print(json.dumps({"layout_sweep": layout_sweep(moe),
                          "unit": "us per moe_dispatch_layout call (kernel time)"}), flush=True)
        return
    w = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    n_phys = w.experts
    rep_off = rep_thr = None
    if args.replicas > 0:
        hot = workloads.popularity(w.experts, w.routing, w.seed)[:args.replicas]
        off_np, thr_np = workloads.replica_plan(w.experts, hot, 4)
        n_phys = int(off_np[-1])
        rep_off = torch.from_numpy(off_np).to(dev)
        rep_thr = torch.from_numpy(thr_np.view("int32")).to(dev)
        rep_ids = torch.empty((w.bs, w.topk), dtype=torch.int32, device=dev)
    cap = moe.moe_dispatch_capacity(w.bs, w.topk, n_phys, w.align)
    fp8_combine = args.combine == "fp8"
    inp = workloads.make(w, rows_y=None if (w.identity_experts or fp8_combine) else cap)
    if fp8_combine:
        yc, ys = workloads.e4m3_rows(cap, w.hidden, w.seed)

    nbytes = algorithmic_bytes(w.bs, w.hidden, n_phys, w.topk, inp["shared"] is not None,
                               fp8=w.fp8, fp8_combine=fp8_combine)
    step_bytes = sum(nbytes.values())
    sets = args.sets or buffer_sets(w, cap, step_bytes, fp8_combine)

    ids = torch.from_numpy(inp["expert_ids"]).to(dev)
    scales = torch.from_numpy(inp["expert_scales"]).to(dev)
    x0 = inp["x"].to(dev)
    y0 = None if (w.identity_experts or fp8_combine) else inp["y"].to(dev)
    yc0 = yc.to(dev) if fp8_combine else None
    ys0 = ys.to(dev) if fp8_combine else None
    sh0 = None if inp["shared"] is None else inp["shared"].to(dev)
    # Every output of every set is written once here (zero-filled), before
    # the warm-up, so that no step writes a buffer for the first time.
    bufs = []
    for i in range(sets):
        ex = torch.zeros((cap, w.hidden), dtype=torch.uint8 if w.fp8 else torch.bfloat16,
                         device=dev)
        bufs.append({
            "index": i,
            "x": x0 if i == 0 else x0.clone(),
            "y": ex if y0 is None else (y0 if i == 0 else y0.clone()),
            "y_codes": None if yc0 is None else (yc0 if i == 0 else yc0.clone()),
            "y_scales": None if ys0 is None else (ys0 if i == 0 else ys0.clone()),
            "scales": (torch.zeros((cap, w.hidden // 128), dtype=torch.float32, device=dev)
                       if w.fp8 else None),
            "shared": None if sh0 is None else (sh0 if i == 0 else sh0.clone()),
            "expand_x": ex,
            "out": torch.zeros((w.bs, w.hidden), dtype=torch.bfloat16, device=dev),
            "layout": moe.Layout(torch.zeros(n_phys, dtype=torch.int32, device=dev),
                                 torch.zeros(n_phys + 1, dtype=torch.int32, device=dev),
                                 torch.zeros(w.bs * w.topk, dtype=torch.int32, device=dev),
                                 torch.zeros(1, dtype=torch.int32, device=dev)),
        })
    ws_bytes = moe.moe_dispatch_layout_workspace_size(w.bs, w.topk, n_phys)
    ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    route_ids = rep_ids if args.replicas > 0 else ids

    rank_offsets = (torch.empty(args.ep + 1, dtype=torch.int32, device=dev) if args.ep
                    else None)

    # Every library call of a step goes through run(): directly, or, while
    # `collect` is a list, as a prepared call (--prepared) appended to it.
    collect = None

    def run(entry, *a, **k):
        if collect is None:
            return entry(*a, **k)
        call = moe.prepare(entry, *a, **k)
        collect.append(call)
        return call.result

    def layout(b):
        if args.ep:
            return run(moe.moe_dispatch_layout_ep, ids, w.experts, args.ep, w.align,
                       out=b["layout"], rank_offsets=rank_offsets, workspace=ws)[0]
        if args.replicas > 0:
            return run(moe.moe_dispatch_layout_replicated,
                       ids, w.experts, rep_off, rep_thr, 1234, w.align, out=b["layout"],
                       replica_ids=rep_ids, workspace=ws)[1]
        return run(moe.moe_dispatch_layout, ids, w.experts, w.align, out=b["layout"],
                   workspace=ws)

    def dispatch(b, lay):
        run(moe.moe_dispatch, b["x"], route_ids, lay.expand_idx, lay.ep_send_counts, n_phys,
            expand_x=b["expand_x"], capacity_rows=cap, out_dtype="fp8" if w.fp8 else "bf16",
            quant_scales=b["scales"])

    def combine(b, lay):
        if fp8_combine:
            run(moe.moe_combine_fp8, b["y_codes"], b["y_scales"], route_ids, lay.expand_idx,
                lay.ep_send_counts, scales, b["shared"], n_phys, out=b["out"])
        else:
            run(moe.moe_combine, b["y"], route_ids, lay.expand_idx, lay.ep_send_counts, scales,
                b["shared"], n_phys, out=b["out"])

    def front(b):
        """Layout and dispatch of one step; returns the layout."""
        if args.fused and args.replicas > 0:
            run(moe.moe_dispatch_fused_replicated,
                b["x"], ids, w.experts, rep_off, rep_thr, 1234, w.align, out=b["layout"],
                replica_ids=rep_ids, capacity_rows=cap, expand_x=b["expand_x"],
                out_dtype="fp8" if w.fp8 else "bf16", quant_scales=b["scales"], workspace=ws)
            return b["layout"]
        if args.fused:
            run(moe.moe_dispatch_fused, b["x"], ids, n_phys, w.align, out=b["layout"],
                capacity_rows=cap, expand_x=b["expand_x"], out_dtype="fp8" if w.fp8 else "bf16",
                quant_scales=b["scales"], workspace=ws)
            return b["layout"]
        lay = layout(b)
        dispatch(b, lay)
        return lay

    def step(b):
        if plans is not None:
            for call in plans[b["index"]]:
                call()
            return
        combine(b, front(b))

    plans = None
    if args.prepared:
        # One prepared call per library call of a step, per buffer set.
        plans = []
        for b in bufs:
            collect = []
            combine(b, front(b))
            plans.append(collect)
        collect = None

    def breakdown_step(b, pairs):
        """One step with every kernel launch taking one of `pairs`; returns
        the pairs taken, in launch order (the combine last), and with the
        layout and dispatch as separate calls the number of launches of the
        layout call (else None)."""
        moe.moe_time_next_launches(pairs)
        cut = None
        if args.fused:
            lay = front(b)
        else:
            lay = layout(b)
            cut = len(pairs) - moe.moe_time_unused_launches()
            dispatch(b, lay)
        combine(b, lay)
        used = len(pairs) - moe.moe_time_unused_launches()
        moe.moe_time_next_launches([])
        return pairs[:used], cut

    def new_pairs(n):
        """n (start, stop) timing-event pairs, each recorded once so that the
        event exists before a launch is bound to it."""
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(n)]
        for a, z in pairs:
            a.record(stream)
            z.record(stream)
        return pairs

    def split_kernels(taken, cut):
        """Kernel times (ms) of one step by role: the combine is the last
        launch; with separate calls the layout call's launches come first and
        the dispatch call's (a read-ahead launch, then the scatter) follow;
        from moe_dispatch_fused, the layout launch then the scatter, or one
        fused kernel."""
        ms = [a.elapsed_time(z) for a, z in taken]
        if cut is not None:
            return {"layout": sum(ms[:cut]), "dispatch": sum(ms[cut:-1]), "combine": ms[-1],
                    "layout_launches": cut, "dispatch_launches": len(ms) - 1 - cut}
        if len(ms) == 2:
            return {"layout+dispatch (fused)": ms[0], "combine": ms[1]}
        return {"layout": sum(ms[:-2]), "dispatch": ms[-2], "combine": ms[-1],
                "layout_launches": len(ms) - 2}

    if args.latency_floor:
        print(json.dumps({"workload": w.name, "latency_floor_us_per_launch": latency_floor(
            moe, w, bufs[0], route_ids, scales, n_phys, cap, front, combine)}), flush=True)
        return

    # Warm-up: at least one step per buffer set, so that every set has run
    # once before the timed region; the steps run are reported as
    # warmup_steps_run.
    warmup_run = max(args.warmup, sets)
    for i in range(warmup_run):
        step(bufs[i % sets])
    torch.cuda.synchronize()

    graphs = None
    per_graph = steps_per_graph(args.steps)
    if not args.eager:
        # Steps are captured per_graph at a time, the way a serving loop
        # replays a whole pass; one graph per distinct sequence of buffer
        # sets.  No call allocates or enqueues a memset when its outputs are
        # given.  Each graph is replayed once before the timed region.
        graphs = []
        for c in range(sets // math.gcd(sets, per_graph)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for j in range(per_graph):
                    step(bufs[(c * per_graph + j) % sets])
            graphs.append(g)
        for g in graphs:
            g.replay()   # counted in warmup_steps_run
        torch.cuda.synchronize()

    # Timed region: exactly K steps on the host clock, synchronised on both
    # sides, with nothing bound to a launch.  Two events recorded on the
    # stream at its ends give the same interval on the GPU's clock (without
    # the host's wake-up after the last kernel).
    region = new_pairs(1)[0]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    region[0].record(stream)
    if graphs is None:
        for i in range(args.steps):
            step(bufs[i % sets])
    else:
        for c in range(args.steps // per_graph):
            graphs[c % len(graphs)].replay()
    region[1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gpu_ms_per_step = region[0].elapsed_time(region[1]) / args.steps

    # Kernel times: ROOFLINE_STEPS eager steps after the timed region, every
    # launch of each bound to its own event pair, stamped with the kernel's
    # own start and end (a bound launch costs its step a few microseconds of
    # host and queue time, which is why none sits inside the timed region).
    # The roofline takes the combine launches of these steps.
    steps_taken = [breakdown_step(bufs[(args.steps + i) % sets], new_pairs(16))
                   for i in range(ROOFLINE_STEPS)]
    torch.cuda.synchronize()
    per_step = [split_kernels(t, cut) for t, cut in steps_taken]
    kern_ms = {r: [d[r] for d in per_step] for r in per_step[0]
               if r not in ("layout_launches", "dispatch_launches")}
    com_ms = kern_ms["combine"]
    mean = lambda v: sum(v) / len(v)

    def pct(v):
        """p10 / median / p90 in microseconds (nearest rank)."""
        o = sorted(v)
        at = lambda q: o[min(len(o) - 1, max(0, round(q * (len(o) - 1))))]
        return [round(at(q) * 1e3, 2) for q in (0.1, 0.5, 0.9)]
    ms_per_step = elapsed * 1e3 / args.steps
    status = int(bufs[0]["layout"].status.cpu()[0])
    if status != 0:
        raise SystemExit(f"layout status flags {status}: routing is invalid")

    combine_s = mean(com_ms) / 1e3
    # When moe_dispatch_fused's layout launch reads the token rows ahead,
    # the dispatch's x reads happen in the layout's time, so the two are
    # rated together: each rate below divides bytes by the time of the
    # kernels that move them.
    read_ahead = args.fused and "layout" in kern_ms
    if read_ahead:
        kern_ms["layout+dispatch"] = [a + b for a, b in zip(kern_ms["layout"],
                                                            kern_ms["dispatch"])]
    role_bytes = {"layout": nbytes["layout"], "combine": nbytes["combine"],
                  "layout+dispatch (fused)": nbytes["layout"] + nbytes["dispatch"],
                  "layout+dispatch": nbytes["layout"] + nbytes["dispatch"]}
    if not read_ahead:
        role_bytes["dispatch"] = nbytes["dispatch"]
    achieved = nbytes["combine"] / combine_s / 1e9
    step_gbs = step_bytes / (ms_per_step / 1e3) / 1e9
    traffic = None if (fp8_combine or args.replicas > 0) else read_traffic(w.name)
    result = {
        "metric": METRIC,
        "value": round(step_gbs, 2),
        "unit": "GB/s",
        "tokens_per_s": round(w.bs / (ms_per_step / 1e3), 1),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warmup_run + (len(graphs) * per_graph if graphs else 0),
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 (dispatch e4m3, fp32 scales)" if w.fp8 else "bf16",
        "arithmetic": ("int32 layout; "
                       + ("e4m3 quantisation in fp32" if w.fp8 else "bf16 bit copies")
                       + " in dispatch; fp32 fused multiply-add chain in combine, "
                         "rounded once to bf16"),
        "data": "synthetic (seeded generators; no routing trace or trained weights)",
        "config": {"workload": w.name, "bs": w.bs, "hidden": w.hidden, "experts": w.experts,
                   "topk": w.topk, "routing": w.routing + (f"(alpha={w.alpha})"
                                                           if w.routing == "zipf" else ""),
                   "align": w.align, "capacity_rows": cap, "buffer_sets": sets,
                   "x_bytes_between_reuse": 2 * w.bs * w.hidden * (sets - 1),
                   "launch": (("eager, prepared calls" if args.prepared else "eager")
                              if args.eager else f"hip graphs of {per_graph} steps"),
                   "layout_dispatch": (("moe_dispatch_fused_replicated" if args.replicas > 0
                                        else "moe_dispatch_fused") if args.fused
                                       else "separate"),
                   "combine_input": "e4m3 + fp32 scales" if fp8_combine else "bf16",
                   "replicas": ({"hot_experts": args.replicas, "per_hot": 4,
                                 "physical": n_phys} if args.replicas > 0 else None),
                   "ep_world_size": args.ep or None,
                   "bytes_per_step": step_bytes},
        "gpu_ms_per_step": round(gpu_ms_per_step, 4),
        "kernel_times": (f"events bound to each launch (kernel start to end) in "
                         f"{ROOFLINE_STEPS} eager steps after the timed region"),
        "layout_launches": per_step[0].get("layout_launches", 0),
        "dispatch_launches": per_step[0].get("dispatch_launches", 1),
        "kernels_ms": {r: round(mean(v), 4) for r, v in kern_ms.items()},
        "kernels_gbs": {r: round(role_bytes[r] / mean(v) / 1e6, 1) for r, v in kern_ms.items()
                        if r in role_bytes},
        "kernels_us_p10_p50_p90": {r: pct(v) for r, v in kern_ms.items()},
        "roofline": {"kernel": "combine_fp8" if fp8_combine else "combine", "bound": "hbm",
                     "timed_launches": len(com_ms),
                     "timing": (f"HIP events bound to every launch (kernel start to end) "
                                f"in {ROOFLINE_STEPS} eager steps after the timed region"),
                     "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "traffic_unit": "HBM bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE)",
                     "algorithmic_bytes_per_launch": nbytes["combine"],
                     "us_p10_p50_p90": pct(com_ms),
                     "step_achieved": round(step_gbs, 1),
                     "step_frac": round(step_gbs / HBM_PEAK_GBS, 4)},
    }
    # The probe models bandwidth-bound sizes (a decode-sized step is launch-
    # latency bound, and a probe of it says nothing) with bf16 rows read by
    # the combine.
    if not (args.no_ceiling or fp8_combine or step_bytes < MALL_BYTES):
        lay0 = bufs[0]["layout"]
        slots = (lay0.ep_send_counts[route_ids.reshape(-1).long()].long()
                 + lay0.expand_idx.long()).view(w.bs, w.topk)
        out_row = w.hidden if w.fp8 else 2 * w.hidden
        ceil = practical_ceiling(moe, w, slots, cap, out_row)
        # The scatter's write rate: its row bytes (e4m3: codes and scales)
        # over its kernel time.
        row_w = out_row + (w.hidden // 128 * 4 if w.fp8 else 0)
        scatter_gbs = w.bs * w.topk * row_w / (mean(kern_ms["dispatch"]) / 1e3) / 1e9 \
            if "dispatch" in kern_ms else None
        result["practical_ceiling"] = {
            "probe": "moe_probe_stream_mix: plain 16-B streaming kernel, same read:write row mix",
            "unit": "GB/s", **ceil,
            "combine_frac_of_random_rows": round(
                achieved / ceil["combine_mix"]["random_rows"], 4),
            "combine_frac_of_layout_rows": round(
                achieved / ceil["combine_mix"]["layout_rows"], 4),
            "dispatch_frac_of_random_rows": round(
                nbytes["dispatch"] / (mean(kern_ms["dispatch"]) / 1e3) / 1e9
                / ceil["dispatch_mix"]["random_rows"], 4) if not args.fused else None,
            "dispatch_frac_of_layout_rows": round(
                nbytes["dispatch"] / (mean(kern_ms["dispatch"]) / 1e3) / 1e9
                / ceil["dispatch_mix"]["layout_rows"], 4) if not args.fused else None,
            "scatter_write_gbs": None if scatter_gbs is None else round(scatter_gbs, 1),
            "scatter_writes_frac_of_layout_rows": None if scatter_gbs is None else round(
                scatter_gbs / ceil["scatter_writes"]["layout_rows"], 4)}
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        cores = min(16, len(os.sched_getaffinity(0)))
        if cores > 1:
            result["cpu_baseline_parallel"] = cpu_baseline(w, args.cpu_seconds / 2, cores)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
