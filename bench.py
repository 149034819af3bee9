#!/usr/bin/env python3
"""Benchmark: RMSNorm-training backward at [131072, 4096] BF16 on one MI355X.

A step is one backward call (dx + dw; main kernel + FP64 fold) of the
non-deterministic mode at T = 131072, H = 4096, x / dy BF16 ~ N(0,1),
w FP32 = 1 + 0.1 N(0,1), eps = 1e-6, inputs resident in HBM. Reported:
whole-call throughput in algorithmic GB/s, us/call, the deterministic mode
and the forward on the same shape, the HBM roofline of the call, and the FP64
CPU oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
One GPU only: --gpus N with N > 1 exits with a message.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X published HBM3E bandwidth
T_HEAD, H_HEAD = 131072, 4096
# The pages' number for this workload, on other hardware: the PR #8848 page, B200 (sm_100a)
# table of every measured row, the new non-deterministic backward at [131072, 4096] BF16
# with FP32 weight ("new us" column). Context for vs_baseline, not a target.
PAGES_BWD_US_B200 = 489.86
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_bwd_131072x4096.json")
# Device code the counters measure; the host-side plan that also decides the
# bytes (chunk count, grids, workspace) is compared separately, so that edits
# to validation code elsewhere in the C ABI do not void the counter summary.
KERNEL_SOURCES = ["rmsn_kernels.hpp", "rmsn_device.hpp", "rmsn_bwd_large.hip", "rmsn_fwd.hip",
                  "rmsn_launch.hpp"]


def bwd_bytes(T, H, w_bytes):
    # read x, dy (2 B each), write dx (2 B) per element; rstd 4T; w; dw 4H
    return 6 * T * H + 4 * T + w_bytes * H + 4 * H


def fwd_bytes(T, H, w_bytes):
    return 4 * T * H + 4 * T + w_bytes * H


def kernel_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "rmsnorm_train_fwd_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def headline_plan():
    """The backward plan of the headline call (host-only query), as a list."""
    import torch

    import rmsnorm_train_fwd_amd as R
    x = torch.empty((T_HEAD, H_HEAD), dtype=torch.bfloat16, device="meta")  # shape only
    p = R.rmsnorm_train_bwd_query(x, False)
    return [p.path, p.chunks, p.subchains, p.fold_group, p.grid, p.fold_grid, p.workspace_bytes]


def measured_traffic():
    """HBM bytes per call from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources and the same headline plan; else
    None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != kernel_hash() or t.get("headline_plan") != headline_plan():
        return None
    return t.get("bytes_per_call")


def time_calls(fn, steps, warmup, torch):
    """Per-call HIP-event times (ms) on the current stream, and wall ms per call."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record()
        fn()
        ends[i].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    ev = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    return ev, wall


def stream_ceiling(x, dy, steps, torch):
    """The practical HBM ceiling beside the kernels: the bandwidth probe
    (probe/librmsn_probe.so, built beside the library) streams the backward's inputs
    in the same tile-dealt pattern with no arithmetic: two read + one written,
    one read + one written, read only. The output is allocated here, after the
    timed calls have freed theirs, so the caching allocator hands it the block
    their dx and y used (the same relative placement, which matters on this
    device). GB/s from the mean of HIP-event times."""
    import ctypes

    path = os.path.join(ROOT, "probe", "librmsn_probe.so")
    if not os.path.exists(path):
        print("[bench] bandwidth probe not built; ceiling omitted", file=sys.stderr, flush=True)
        return None
    f = ctypes.CDLL(path).rmsn_stream_probe
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    f.restype = ctypes.c_int
    nbytes = x.numel() * x.element_size()
    assert dy.numel() * dy.element_size() == nbytes and x.is_contiguous() and dy.is_contiguous()
    out = torch.empty_like(x)
    stream = torch.cuda.current_stream().cuda_stream
    out_ = {"by_pattern": {"dealt": {}, "oneshot": {}, "oneshot_vec1": {}}}
    for nin, key, moved in ((2, "r2w1_GBps", 3 * nbytes), (1, "r1w1_GBps", 2 * nbytes),
                            (0, "r1_GBps", nbytes)):
        for pattern, name in ((0, "dealt"), (1, "oneshot"), (2, "oneshot_vec1")):
            def call():
                rc = f(nin, pattern, x.data_ptr(), dy.data_ptr(), out.data_ptr(), nbytes, 256,
                       stream)
                if rc != 0:
                    raise RuntimeError(f"bandwidth probe failed: hip error {rc}")
            ev, _ = time_calls(call, steps, 3, torch)
            out_["by_pattern"][name][key] = round(moved / (sum(ev) / len(ev) * 1e-3) / 1e9, 1)
        out_[key] = max(v[key] for v in out_["by_pattern"].values())
    out_["probe"] = ("the backward's x and dy, 16-byte non-temporal accesses, no arithmetic; "
                     "dealt: 256 workgroups x 1024 threads, 16 KiB tiles dealt in turn, next "
                     "tile's loads in flight (the kernels' pattern); oneshot: one 256-thread "
                     "workgroup per 16 KiB tile, 4 vectors per thread; oneshot_vec1: one "
                     "256-thread workgroup per 4 KiB, one vector per thread; the ceiling is the "
                     "fastest of the three")
    return out_


def cpu_baseline(p, rows_sample, reps=3):
    """The FP64 oracle (plain C, unchanged) on the workload's rows, median of
    reps: once on one thread, and once on every core this process may use, the
    rows cut into one fixed block per core, each block a concurrent call of the
    same single-threaded oracle (ctypes releases the GIL for the call), and the
    blocks' dw added in block order. The single-threaded call stays the
    checker; the blocked run only times the oracle on all cores."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch

    import oracle

    W = p.width
    xs = p.x.view(-1, W)[:rows_sample].contiguous().view(torch.int16).numpy().view(np.uint16)
    dys = p.dy.view(-1, W)[:rows_sample].contiguous().view(torch.int16).numpy().view(np.uint16)
    w64 = p.w.double().numpy()
    host = host_cpu()
    cores = host["cpus_available"]
    bounds = [rows_sample * i // cores for i in range(cores + 1)]
    oracle.lib()  # load (and, if stale, build) the library before anything is timed

    def one_thread():
        oracle.bwd(oracle.View.dense(dys), oracle.View.dense(xs), w64, p.eps)

    def block(i):
        a, b = bounds[i], bounds[i + 1]
        return oracle.bwd(oracle.View.dense(dys[a:b]), oracle.View.dense(xs[a:b]), w64, p.eps)

    def all_cores(ex):
        dw = np.zeros(W)
        for _, dwb in ex.map(block, range(cores)):
            dw = dw + dwb
        return dw

    def med_time(fn):
        times = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            times.append(time.perf_counter() - t0)
        return sorted(times)[len(times) // 2]

    dt1 = med_time(one_thread)
    with ThreadPoolExecutor(cores) as ex:
        dtn = med_time(lambda: all_cores(ex))
    nbytes = bwd_bytes(rows_sample, W, 4)
    scale = p.T / rows_sample
    return {
        "value": round(nbytes / dtn / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
        "sample": f"backward (dx for every row, dw over every row) of {rows_sample} of {p.T} "
                  f"rows, width {W}, FP64 C oracle unchanged: {cores} concurrent calls on fixed "
                  f"row blocks (dw added in block order), median of {reps} runs ({dtn:.2f} s "
                  "each); same algorithmic byte model as value",
        "us_per_call": round(dtn * 1e6 * scale, 1),
        "single_thread": {"value": round(nbytes / dt1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                          "us_per_call": round(dt1 * 1e6 * scale, 1),
                          "sample": f"the same rows in one call, median of {reps} runs "
                                    f"({dt1:.2f} s each)"},
        "host": host,
    }


def host_cpu():
    """CPU model (lscpu, else /proc/cpuinfo) and the logical CPUs this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    lscpu = {}
    try:
        import subprocess

        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        for line in out.splitlines():
            k, _, v = line.partition(":")
            if k.strip() in ("Model name", "Vendor ID", "CPU(s)", "Thread(s) per core",
                             "Core(s) per socket", "Socket(s)", "NUMA node(s)", "CPU max MHz",
                             "L3 cache", "Hypervisor vendor", "Virtualization type"):
                lscpu[k.strip()] = v.strip()
    except (OSError, ValueError, subprocess.SubprocessError):
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = os.cpu_count()
    return {"model": lscpu.get("Model name", model), "cpus_available": avail, "lscpu": lscpu}


def cpu_sweep(out_md, reps=3):
    """The FP64 oracle (plain C, unchanged) timed on every workload of the
    configurations, on one thread and on every core (the sampled rows cut into
    one block of tokens per core, each block a concurrent call of the same
    single-threaded oracle): each call runs on a sample of at most 2^24
    elements of the workload's rows (the oracle's cost is linear in the row
    count), median of reps, scaled to the full row count. Writes a markdown
    table."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch

    import oracle
    import synth

    cores = host_cpu()["cpus_available"]
    pool = ThreadPoolExecutor(cores)
    oracle.lib()  # load (and, if stale, build) the library before anything is timed

    def bits(t):
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)

    def med_time(fn):
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return sorted(ts)[len(ts) // 2]

    rows_out = []

    def add(cfg, workload, op, rows, sample_rows, dt, dtn, nbytes):
        us = dt * 1e6 * rows / sample_rows
        usn = dtn * 1e6 * rows / sample_rows
        rows_out.append((cfg, workload, op, sample_rows, dt, us, nbytes / (us * 1e-6) / 1e9, usn,
                         nbytes / (usn * 1e-6) / 1e9))
        print(f"[cpu] {cfg:3s} {workload:32s} {op:4s} {us:14.1f} us  all cores {usn:12.1f} us",
              file=sys.stderr, flush=True)

    def views(p, form, t0=0, t1=None):
        """The problem's views, or those of tokens [t0, t1) only."""
        t1 = p.T if t1 is None else t1

        def v(buf):
            b = bits(buf)[t0 * p.row_stride:]
            return oracle.View(b, t1 - t0, p.heads, p.width, p.row_stride, p.head_stride)
        return v(p.x), v(p.dy), (v(p.extra) if form != "plain" else None), \
            (v(p.dh) if form == "residual" else None)

    def both(p, form, call):
        """Median times of call(x, dy, e, dh) on all rows, and on one block of
        tokens per core run concurrently."""
        dt = med_time(lambda: call(*views(p, form)))
        nb = min(cores, p.T)
        cuts = [p.T * i // nb for i in range(nb + 1)]
        blocks = [views(p, form, cuts[i], cuts[i + 1]) for i in range(nb)]
        dtn = med_time(lambda: list(pool.map(lambda b: call(*b), blocks)))
        return dt, dtn

    def run(cfg, T, W, heads=1, rs=None, hs=None, form="plain", w_dtype="f32", ops=("fwd", "bwd"),
            label=None):
        rows = T * heads
        ts = max(1, min(T, (1 << 24) // (W * heads)))
        p = synth.make(ts, W, seed=0, heads=heads, w_dtype=w_dtype, form=form, row_stride=rs,
                       head_stride=hs)
        w = p.w.double().numpy()
        wb = 4 if w_dtype == "f32" else 2
        n, sr = rows * W, ts * heads
        name = label or f"[{T},{W}]"
        if "fwd" in ops:
            if form == "plain":
                dt, dtn = both(p, form, lambda x, dy, e, dh: oracle.fwd(x, w, p.eps))
                add(cfg, name, "fwd", rows, sr, dt, dtn, 4 * n + 4 * rows + wb * W)
            elif form == "residual":
                dt, dtn = both(p, form, lambda x, dy, e, dh: oracle.res_fwd(x, e, w, p.eps))
                add(cfg, name, "fwd", rows, sr, dt, dtn, 8 * n + 4 * rows + wb * W)
            else:
                dt, dtn = both(p, form, lambda x, dy, e, dh: oracle.gate_fwd(x, e, w, p.eps))
                add(cfg, name, "fwd", rows, sr, dt, dtn, 6 * n + 4 * rows + wb * W)
        if "bwd" in ops:
            if form == "plain":
                dt, dtn = both(p, form, lambda x, dy, e, dh: oracle.bwd(dy, x, w, p.eps))
                add(cfg, name, "bwd", rows, sr, dt, dtn, 6 * n + 4 * rows + wb * W + 4 * W)
            elif form == "residual":
                dt, dtn = both(p, form, lambda x, dy, e, dh: oracle.bwd(dy, x, w, p.eps, dh=dh))
                add(cfg, name, "bwd", rows, sr, dt, dtn, 8 * n + 4 * rows + wb * W + 4 * W)
            else:
                dt, dtn = both(p, form, lambda x, dy, e, dh: oracle.gate_bwd(dy, x, e, w, p.eps))
                add(cfg, name, "bwd", rows, sr, dt, dtn, 10 * n + 4 * rows + wb * W + 4 * W)

    run("1", 8, 512, w_dtype="bf16")
    for W in (512, 1536, 2048, 4096, 5120, 6144):
        run("2", 203, W, ops=("bwd",))
    for rs_, hs_ in ((12288, 512), (6144, 256)):
        run("2", 203, 256, heads=24, rs=rs_, hs=hs_, ops=("bwd",),
            label=f"[203,24,256] strides ({rs_},{hs_},1)")
    for W in (1536, 2048, 4096, 5120, 6144):
        run("3", 131072, W)
    run("4", 131072, 6144, form="residual", label="[131072,6144] residual")
    for T in (3534, 8192, 16384):
        run("5", T, 4096, form="gate", label=f"[{T},4096] gate")
    pool.shutdown()
    host = host_cpu()
    lines = ["# FP64 CPU oracle on every workload (one thread and all cores)", "",
             "Command (repository root $REPO, on the MI355X host; committed files only):", "",
             "```", "python3 $REPO/bench.py --cpu-sweep <this file>", "```", "",
             f"Host: {host['model']} (lscpu: "
             f"{'; '.join(f'{k} {v}' for k, v in host['lscpu'].items())}), "
             f"{host['cpus_available']} logical CPUs "
             "available. The oracle is the plain single-threaded C, unchanged: timed on one "
             f"thread, and on all {cores} cores as one block of tokens per core, each block a "
             "concurrent call of the same oracle (ctypes releases the GIL). Each call runs on a "
             "sample of at most 2^24 elements of the workload's rows, median of "
             f"{reps} runs, and is scaled to the full row count (the oracle's cost is linear in "
             "the rows). GB/s uses the same algorithmic bytes as the GPU tables: fwd 4TH, bwd "
             "6TH, residual 8TH each way, gate fwd 6TH and bwd 10TH (+ per-row and per-column "
             "terms).", "",
             "| cfg | workload | op | rows timed | s per sample (1 thread) | us per full call, 1 "
             f"thread | GB/s, 1 thread | us per full call, {cores} cores | GB/s, {cores} cores |",
             "|---|---|---|---|---|---|---|---|---|"]
    for cfg, wl, op, sr, dt, us, gbps, usn, gbpsn in rows_out:
        lines.append(f"| {cfg} | {wl} | {op} | {sr} | {dt:.4f} | {us:.1f} | {gbps:.3f} | "
                     f"{usn:.1f} | {gbpsn:.3f} |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


GATE_TS = (16384, 8192, 3534)  # gated form measured by the counter runs: [T, 4096], in this order
SWEEP_REPS = 80  # calls per case and process in --sweep (the pages take 4 x 20 per process)


def traffic_probe():
    """For rocprofv3 --pmc runs: one plain copy of known size (calibration),
    then three forward and three backward calls at the headline shape, and
    three gated forward and backward calls at each of [16384 | 8192 | 3534, 4096]."""
    import torch

    import rmsnorm_train_fwd_amd as R
    import synth

    dev = torch.device("cuda:0")
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)  # 1 GiB read + 1 GiB written
    torch.cuda.synchronize()
    del src, dst
    p = synth.make(T_HEAD, H_HEAD, seed=0, w_dtype="f32")
    x = p.x.to(dev).view(T_HEAD, H_HEAD)
    dy = p.dy.to(dev).view(T_HEAD, H_HEAD)
    w = p.w.to(dev)
    for _ in range(3):
        _, rstd = R.rmsnorm_train_fwd(x, w, p.eps)
    for _ in range(3):
        R.rmsnorm_train_bwd(dy, x, rstd, w, False)
    torch.cuda.synchronize()
    del x, dy, rstd
    for T in GATE_TS:
        g = synth.make(T, H_HEAD, seed=0, w_dtype="f32", form="gate")
        x, z = g.x.to(dev).view(T, H_HEAD), g.extra.to(dev).view(T, H_HEAD)
        dy, w = g.dy.to(dev).view(T, H_HEAD), g.w.to(dev)
        for _ in range(3):
            _, rstd = R.rmsnorm_silu_gate_train_fwd(x, z, w, g.eps)
        for _ in range(3):
            R.rmsnorm_silu_gate_train_bwd(dy, x, z, rstd, w, False)
        torch.cuda.synchronize()
        del x, z, dy, w, rstd
    print("[bench] traffic probe done", file=sys.stderr, flush=True)


def sweep(out_path, reps=SWEEP_REPS):
    """Every workload of the build, one graph-replayed call per timing with a
    512 MB write between calls (cold L2 and Infinity Cache). Writes a markdown
    table to out_path and returns the rows."""
    import torch

    import rmsnorm_train_fwd_amd as R
    import synth

    dev = torch.device("cuda:0")
    # Cold caches: read (not write) 512 MB between calls, evicting L2 and the
    # 256 MB Infinity Cache without leaving dirty lines whose write-back would
    # land inside the timed call.
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)  # FP32 sum: one read pass, no cast

    def graph_time(fn):
        fn()  # allocations (outputs, workspace) happen outside capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        ts = []
        # a marker range per case lets a rocprofv3 --marker-trace run attribute
        # the kernels of these replays to this case (bench.py --sweep-kernels)
        torch.cuda.nvtx.range_push(f"rmsn_case_{len(rows)}")
        for _ in range(reps):
            flush.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b) * 1e3)
        torch.cuda.nvtx.range_pop()
        ts.sort()
        return ts[len(ts) // 2]

    rows = []

    def add(cfg, shape, op, us, nbytes):
        gbps = nbytes / (us * 1e-6) / 1e9 if nbytes else None
        rows.append((cfg, shape, op, us, gbps))
        pct = f"{100 * gbps / HBM_PEAK_GBPS:.1f}%" if gbps else "-"
        print(f"[sweep] {cfg:4s} {shape:34s} {op:26s} {us:9.2f} us  "
              f"{(f'{gbps:7.0f} GB/s' if gbps else ''):>12s} {pct}", file=sys.stderr, flush=True)

    def run_plain(cfg, T, H, w_dtype, modes, heads=1, rs=None, hs=None, fwd=True, label=None):
        p = synth.make(T, H, seed=0, heads=heads, w_dtype=w_dtype, row_stride=rs, head_stride=hs)
        wb = 4 if w_dtype == "f32" else 2
        x = p.x.to(dev).as_strided(*((p.T, p.width), (p.row_stride, 1)) if heads == 1 else
                                    ((p.T, heads, p.width), (p.row_stride, p.head_stride, 1)))
        dy = p.dy.to(dev).as_strided(x.shape, x.stride())
        w = p.w.to(dev)
        y, rstd = R.rmsnorm_train_fwd(x, w, p.eps)
        rws = p.rows
        shape = label or f"[{T},{H}] w {w_dtype}"
        if fwd:
            add(cfg, shape, "fwd", graph_time(lambda: R.rmsnorm_train_fwd(x, w, p.eps)),
                fwd_bytes(rws, H, wb))
        for det in modes:
            plan = R.rmsnorm_train_bwd_query(x, det, dy=dy)
            ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device=dev)
            path = "small" if plan.path == R.PATH_SMALL else "large"
            add(cfg, shape, f"bwd {'det' if det else 'nondet'} ({path})",
                graph_time(lambda: R.rmsnorm_train_bwd(dy, x, rstd, w, det, workspace=ws)),
                bwd_bytes(rws, H, wb))

    tiny = torch.zeros(1, device=dev)
    add("-", "launch floor: 1-element kernel", "graph replay", graph_time(lambda: tiny.add_(1)), 0)
    run_plain("1", 8, 512, "bf16", [True], label="[8,512] w bf16")
    for H in (512, 1536, 2048, 4096, 5120, 6144):
        for T in (1, 8, 32, 128, 203):
            for wd in ("f32", "bf16"):
                run_plain("2", T, H, wd, [True], fwd=False)
    for T in (1, 32, 203):
        for (rs, hs) in ((12288, 512), (6144, 256)):
            run_plain("2", T, 256, "f32", [True], heads=24, rs=rs, hs=hs, fwd=False,
                      label=f"[{T},24,256] strides ({rs},{hs},1)")
    for H in (1536, 2048, 4096, 5120, 6144):
        for T in (65537, 98304, 131072):
            run_plain("3", T, H, "f32", [False, True])
            torch.cuda.empty_cache()
    # fused residual, width 6144
    for T in (32, 65537, 131072):
        for wd in ("bf16", "f32"):
            p = synth.make(T, 6144, seed=0, w_dtype=wd, form="residual")
            wb = 4 if wd == "f32" else 2
            x, res = p.x.to(dev).view(T, 6144), p.extra.to(dev).view(T, 6144)
            dy, dh = p.dy.to(dev).view(T, 6144), p.dh.to(dev).view(T, 6144)
            w = p.w.to(dev)
            y, rstd, h = R.rmsnorm_train_fwd(x, w, p.eps, residual=res)
            shape = f"[{T},6144] residual w {wd}"
            add("4", shape, "fwd", graph_time(lambda: R.rmsnorm_train_fwd(x, w, p.eps, residual=res)),
                8 * T * 6144 + 4 * T + wb * 6144)
            for det in (False, True):
                plan = R.rmsnorm_train_bwd_query(h, det)
                ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device=dev)
                add("4", shape, f"bwd {'det' if det else 'nondet'}",
                    graph_time(lambda: R.rmsnorm_train_bwd(dy, h, rstd, w, det, dh=dh, workspace=ws)),
                    8 * T * 6144 + 4 * T + wb * 6144 + 4 * 6144)
            del x, res, dy, dh, y, h
            torch.cuda.empty_cache()
    # SiLU gate, width 4096: fwd, bwd, checkpointed step (fwd, fwd recompute, bwd)
    for T in (3534, 8192, 16384):
        p = synth.make(T, 4096, seed=0, w_dtype="f32", form="gate")
        x, z = p.x.to(dev).view(T, 4096), p.extra.to(dev).view(T, 4096)
        dy = p.dy.to(dev).view(T, 4096)
        w = p.w.to(dev)
        y, rstd = R.rmsnorm_silu_gate_train_fwd(x, z, w, p.eps)
        shape = f"[{T},4096] gate w f32"
        fb, bb = 6 * T * 4096 + 4 * T + 4 * 4096, 10 * T * 4096 + 4 * T + 8 * 4096
        add("5", shape, "fwd", graph_time(lambda: R.rmsnorm_silu_gate_train_fwd(x, z, w, p.eps)), fb)
        for det in (False, True):
            plan = R.rmsnorm_train_bwd_query(x, det)
            ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device=dev)
            add("5", shape, f"bwd {'det' if det else 'nondet'}", graph_time(
                lambda: R.rmsnorm_silu_gate_train_bwd(dy, x, z, rstd, w, det, workspace=ws)), bb)

            def step():
                R.rmsnorm_silu_gate_train_fwd(x, z, w, p.eps)
                _, r2 = R.rmsnorm_silu_gate_train_fwd(x, z, w, p.eps)
                R.rmsnorm_silu_gate_train_bwd(dy, x, z, r2, w, det, workspace=ws)
            add("5", shape, f"step 2xfwd+bwd {'det' if det else 'nondet'}", graph_time(step),
                2 * fb + bb)
    # next, rank 2: the grouped per-head SiLU gate at the five tokens x heads shapes
    # of the gated page's Table 1; head dim 256 stands in for the unstated one
    for T, heads in ((3534, 48), (4097, 48), (6000, 48), (7684, 48), (8192, 32)):
        W = 256
        p = synth.make(T, W, seed=0, heads=heads, w_dtype="f32", form="gate")
        shp = ((T, heads, W), (heads * W, W, 1))
        x, z = p.x.to(dev).as_strided(*shp), p.extra.to(dev).as_strided(*shp)
        dy = p.dy.to(dev).as_strided(*shp)
        w = p.w.to(dev)
        y, rstd = R.rmsnorm_silu_gate_train_fwd(x, z, w, p.eps)
        rws = T * heads
        shape = f"[{T},{heads},{W}] gate w f32"
        fb, bb = 6 * rws * W + 4 * rws + 4 * W, 10 * rws * W + 4 * rws + 8 * W
        add("n2", shape, "fwd", graph_time(lambda: R.rmsnorm_silu_gate_train_fwd(x, z, w, p.eps)), fb)
        for det in (False, True):
            plan = R.rmsnorm_train_bwd_query(x, det)
            ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device=dev)
            add("n2", shape, f"bwd {'det' if det else 'nondet'}", graph_time(
                lambda: R.rmsnorm_silu_gate_train_bwd(dy, x, z, rstd, w, det, workspace=ws)), bb)
        del x, z, dy, y, rstd
        torch.cuda.empty_cache()
    # next, rank 1: per-head views of width 256 at large row counts
    for T in (4096, 16384, 65536):
        for heads, rs, hs in ((24, 12288, 512), (24, 6144, 256), (4, 1024, 256)):
            run_plain("n1", T, 256, "f32", [False, True], heads=heads, rs=rs, hs=hs,
                      label=f"[{T},{heads},256] strides ({rs},{hs},1)")
            torch.cuda.empty_cache()
    # one GPU's share of the [131072, 4096] call when its rows are split over 4 or 8
    # GPUs (row-sharded data parallelism; the 2-GPU share is config 3's T = 65537)
    for T in (32768, 16384):
        run_plain("e", T, 4096, "f32", [False, True])
        torch.cuda.empty_cache()
    with open(out_path, "w") as fh:
        fh.write("| cfg | workload | op | us/call | algorithmic GB/s | % of 8 TB/s |\n|---|---|---|---|---|---|\n")
        for cfg, shape, op, us, gbps in rows:
            fh.write(f"| {cfg} | {shape} | {op} | {us:.2f} | {f'{gbps:.0f}' if gbps else '-'} | "
                     f"{f'{100 * gbps / HBM_PEAK_GBPS:.1f}' if gbps else '-'} |\n")
    with open(out_path + ".json", "w") as fh:
        json.dump([{"case": i, "cfg": c, "workload": sh, "op": op, "event_us": us,
                    "bytes": (None if g is None else g * us * 1e3)}
                   for i, (c, sh, op, us, g) in enumerate(rows)], fh)
    return rows


def sweep_spans(sweep_json, trace_dir):
    """Kernel-active spans (ns) per case of one rocprofv3 --kernel-trace
    --marker-trace run of --sweep: per marker range (one case), the dispatches
    of this library between two cache-flush dispatches form one replay; its
    span runs from the first start to the last end. Returns {(cfg, workload,
    op): (spans, event_us, bytes)} in case order."""
    import csv
    import glob

    cases = json.load(open(sweep_json))
    kt = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    mt = glob.glob(os.path.join(trace_dir, "**", "*marker_api_trace.csv"), recursive=True)
    if not kt or not mt:
        raise SystemExit(f"no kernel/marker trace under {trace_dir}")
    kern = sorted(((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"])
                   for r in csv.DictReader(open(kt[0]))))
    ranges = {}
    for r in csv.DictReader(open(mt[0])):
        msg = r.get("Message") or r.get("Function") or ""
        if msg.startswith("rmsn_case_"):
            ranges[int(msg.split("_")[-1])] = (int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
    out = {}
    for c in cases:
        if c["case"] not in ranges or c["cfg"] == "-":
            continue
        t0, t1 = ranges[c["case"]]
        spans, folds, cur = [], [], None

        def close(cur):
            spans.append(cur[1] - cur[0])
            folds.append(cur[2])

        for s_, e_, name in kern:
            if s_ < t0 or s_ > t1:
                continue
            if "rmsn::" not in name:  # the cache-flush read between replays
                if cur:
                    close(cur)
                cur = None
            else:
                fold = e_ - s_ if "k_fold" in name else 0
                cur = (s_, e_, fold) if cur is None else (cur[0], max(cur[1], e_), cur[2] + fold)
        if cur:
            close(cur)
        if spans:
            out[(c["cfg"], c["workload"], c["op"])] = (spans, c["event_us"], c["bytes"], folds)
    return out


def sweep_kernels(args, out_md):
    """Markdown table of kernel-active time per call for every workload from
    one or more traced --sweep runs (separate processes): median over all
    calls of all runs, p10-p90, and each run's own median (an A/A check: the
    same case measured again in another process)."""
    if len(args) < 2 or len(args) % 2:
        raise SystemExit("--sweep-kernels takes SWEEP.md.json TRACE_DIR pairs, then OUT.md")
    runs = [sweep_spans(args[i], args[i + 1]) for i in range(0, len(args), 2)]
    n = len(runs)
    names = "abcdefgh"[:n]
    pairs = " ".join(f"$OUT/sweep_{k}.md.json $OUT/prof_sweep_{k}"
                     for k in names)
    out = ["# Every workload: kernel-active time per call, cold caches (rocprofv3)", "",
           "Commands (repository root $REPO, output directory $OUT, on an MI355X; committed files only), "
           f"{n} separate process{'es' if n > 1 else ''}, k = {', '.join(names)}:",
           "", "```", "cd /tmp && export TMPDIR=/tmp",
           "rocprofv3 --kernel-trace --marker-trace --output-format csv -d $OUT/prof_sweep_<k> "
           "-o sweep -- python3 $REPO/bench.py --sweep $OUT/sweep_<k>.md",
           f"python3 $REPO/bench.py --sweep-kernels {pairs} <this file>", "```", "",
           "Each call is one graph replay after a 512 MB read that evicts L2 and the Infinity Cache. "
           "Kernel-active span = first kernel start to last kernel end of the call (all of this "
           "library's kernels of the call: main + fold on the large path). The median and p10-p90 "
           f"run over all calls of all {n} process{'es' if n > 1 else ''} ({SWEEP_REPS} calls "
           "each, the pages' 4 x 20 in one session); the "
           "per-process medians are the A/A check (the same case measured in another process, "
           "where the caching allocator may place the tensors elsewhere). The event column is "
           "the HIP-event time around the replay (median of the processes), which carries a ~13 "
           "us floor on this system. GB/s uses the algorithmic bytes and the median: fwd 4TH, bwd "
           "6TH, residual 8TH each way, gate fwd 6TH and bwd 10TH (+ per-row and per-column "
           "terms). The fold column is the median duration of the k_fold kernel inside the span "
           "(large path only; the small path is one kernel).", "",
           "| cfg | workload | op | kernel-active us/call (median) | p10-p90 | per-process medians "
           "| of which k_fold | algorithmic GB/s | % of 8 TB/s | event us/call |",
           "|---|---|---|---|---|---|---|---|---|---|"]
    for key in runs[0]:
        if not all(key in r for r in runs):
            continue
        allspans = sorted(x for r in runs for x in r[key][0])
        med = allspans[len(allspans) // 2] / 1e3
        p10 = allspans[len(allspans) // 10] / 1e3
        p90 = allspans[(9 * len(allspans)) // 10] / 1e3
        per = [sorted(r[key][0])[len(r[key][0]) // 2] / 1e3 for r in runs]
        ev = sorted(r[key][1] for r in runs)[n // 2]
        nbytes = runs[0][key][2]
        gbps = nbytes / (med * 1e3) if nbytes else None
        folds = sorted(x for r in runs for x in r[key][3])
        fold = folds[len(folds) // 2] / 1e3
        cfg, wl, op = key
        out.append(f"| {cfg} | {wl} | {op} | {med:.2f} | {p10:.2f}-{p90:.2f} | "
                   f"{' / '.join(f'{v:.2f}' for v in per)} | "
                   f"{f'{fold:.2f}' if fold else '-'} | "
                   f"{f'{gbps:.0f}' if gbps else '-'} | "
                   f"{f'{100 * gbps / HBM_PEAK_GBPS:.1f}' if gbps else '-'} | {ev:.2f} |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(out) + "\n")
    print("\n".join(out))


def stats_report(stats_csv, out_md, command):
    """Markdown table of a rocprofv3 --stats kernel summary, with algorithmic
    GB/s for the headline kernels."""
    import csv

    lines = ["# rocprofv3 kernel statistics: backward and forward at [131072, 4096] BF16 (w FP32)",
             "", "Command (repository root $REPO, output directory $OUT, on an MI355X; committed files only):", "",
             "```", "cd /tmp && export TMPDIR=/tmp", command,
             f"python3 $REPO/bench.py --stats-report <run_kernel_stats.csv> <this file>", "```", "",
             f"Algorithmic bytes: backward call {bwd_bytes(T_HEAD, H_HEAD, 4):,} B; forward "
             f"{fwd_bytes(T_HEAD, H_HEAD, 4):,} B.", "",
             "| kernel | calls | avg us | min us | max us | algorithmic GB/s (avg) |",
             "|---|---|---|---|---|---|"]
    for r in csv.DictReader(open(stats_csv)):
        n = r["Name"].strip('"')
        avg = float(r["AverageNs"]) / 1e3
        gb = ""
        if "k_bwd_large" in n:
            gb = f"{bwd_bytes(T_HEAD, H_HEAD, 4) / (avg * 1e-6) / 1e9:.0f} (main kernel alone)"
        elif "k_fwd" in n:
            gb = f"{fwd_bytes(T_HEAD, H_HEAD, 4) / (avg * 1e-6) / 1e9:.0f}"
        elif "k_stream" in n:
            # bandwidth probe over the bench's tensors: k_stream<nin> moves (nin + 1)
            # tensors of T*H BF16 (nin = 0: one, read only)
            nin = int(n.split("<")[1][0])
            moved = (nin + 1) * 2 * T_HEAD * H_HEAD
            gb = f"{moved / (avg * 1e-6) / 1e9:.0f} (probe, {nin or 1} read{'s' if nin == 2 else ''}" \
                 f"{', 1 written' if nin else ''})"
        lines.append(f"| `{n}` | {r['Calls']} | {avg:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {gb} |")
    lines += ["", "k_bwd_large template arguments: <width, FP32 weight, form (0 = plain), "
              "deterministic, rows per batch>. One backward call = k_bwd_large + k_fold.",
              "k_stream / k_stream_oneshot / k_stream_vec1: the bandwidth probe "
              "(probe/librmsn_probe.so) over the same tensors, no arithmetic: the dealt-tile "
              "pattern of the kernels, a one-shot pattern with 4 vectors per thread and one with "
              "one vector per thread; <nin> = tensors read (0 = read only, nothing written)."]
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def traffic_report(fetch_dir, write_dir, out_json, out_md):
    """Calibrated HBM bytes per backward call from two rocprofv3 --pmc runs of
    --traffic-probe (FETCH_SIZE, then WRITE_SIZE), scaled by the readings for
    the 1 GiB device-to-device copy of known size."""
    import csv
    import glob

    def load(d):
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
        return sorted(csv.DictReader(open(f)), key=lambda r: int(r["Dispatch_Id"]))

    F, W = load(fetch_dir), load(write_dir)
    GiB = 1 << 30

    def copy_kib(rows):
        v = [float(r["Counter_Value"]) for r in rows
             if "copyBuffer" in r["Kernel_Name"] and r["Grid_Size"] == str(GiB // 8192)]
        return v[0]

    ff, wf = GiB / (copy_kib(F) * 1024), GiB / (copy_kib(W) * 1024)

    def per(rows, key, factor, part=None):
        """Mean bytes per dispatch of the kernels whose name holds key; part =
        (i, n): the i-th of n equal consecutive groups of those dispatches."""
        v = [float(r["Counter_Value"]) * 1024 * factor for r in rows if key in r["Kernel_Name"]]
        if part is not None:
            i, n = part
            m = len(v) // n
            v = v[i * m:(i + 1) * m]
        return sum(v) / len(v)

    plain_bwd = f"k_bwd_large<{H_HEAD}, true, 0, false"
    kr, kw = per(F, plain_bwd, ff), per(W, plain_bwd, wf)
    plain_fwd, gate_fwd = f"k_fwd<{H_HEAD}, true, 0,", f"k_fwd<{H_HEAD}, true, 2,"
    gate_bwd = f"k_bwd_large<{H_HEAD}, true, 2, false"
    fwr, fww = per(F, plain_fwd, ff), per(W, plain_fwd, wf)
    alg_fwd = fwd_bytes(T_HEAD, H_HEAD, 4)
    import torch
    import rmsnorm_train_fwd_amd as R

    def chunks_of(T):
        return R.rmsnorm_train_bwd_query(torch.empty((T, H_HEAD), dtype=torch.bfloat16,
                                                     device="meta"),
                                         False).chunks

    chunks = chunks_of(T_HEAD)
    # every backward call above ends with one fold; at these shapes all of
    # them fold the same 256 x 4096 partials
    fr, fw = per(F, "k_fold", ff), per(W, "k_fold", wf)
    gate = []
    for i, T in enumerate(GATE_TS):
        GH = T * H_HEAD
        part = (i, len(GATE_TS))
        gfr, gfw = per(F, gate_fwd, ff, part), per(W, gate_fwd, wf, part)
        gbr, gbw = per(F, gate_bwd, ff, part), per(W, gate_bwd, wf, part)
        alg_gf, alg_gb = 6 * GH + 4 * T + 4 * H_HEAD, 10 * GH + 4 * T + 8 * H_HEAD
        part_b = 2 * chunks_of(T) * H_HEAD * 8  # partials written by the main kernel, read by the fold
        gate.append(dict(T=T, fr=gfr, fw=gfw, br=gbr, bw=gbw, alg_f=alg_gf, alg_b=alg_gb,
                         partials=part_b))
    total, alg = kr + kw + fr + fw, bwd_bytes(T_HEAD, H_HEAD, 4)
    out = {"kernel_hash": kernel_hash(), "headline_plan": headline_plan(),
           "workload": "rmsnorm_train_bwd non-deterministic [131072,4096] BF16, w FP32",
           "bytes_per_call": round(total), "algorithmic_bytes_per_call": alg,
           "ratio_to_algorithmic": round(total / alg, 5), "fetch_scale": round(ff, 6),
           "write_scale": round(wf, 6), "k_bwd_large": {"read": round(kr), "write": round(kw)},
           "k_fold": {"read": round(fr), "write": round(fw)},
           "forward": {"workload": "rmsnorm_train_fwd [131072,4096] BF16, w FP32",
                       "read": round(fwr), "write": round(fww), "algorithmic": alg_fwd,
                       "ratio_to_algorithmic": round((fwr + fww) / alg_fwd, 5)},
           "gate": [{"T": g["T"], "width": H_HEAD, "w": "FP32",
                     "forward": {"read": round(g["fr"]), "write": round(g["fw"]),
                                 "algorithmic": g["alg_f"],
                                 "ratio_to_algorithmic": round((g["fr"] + g["fw"]) / g["alg_f"], 5)},
                     "backward": {"read": round(g["br"] + fr), "write": round(g["bw"] + fw),
                                  "algorithmic": g["alg_b"],
                                  "ratio_to_algorithmic":
                                      round((g["br"] + g["bw"] + fr + fw) / g["alg_b"], 5),
                                  "fp64_partials_round_trip": g["partials"]}}
                    for g in gate],
           "calibration_kib": {"fetch": copy_kib(F), "write": copy_kib(W)}}
    with open(out_json, "w") as fh:
        json.dump(out, fh, indent=1)
    gate_rows = "\n".join(
        f"| k_fwd<4096, w FP32, gate> [{g['T']}, 4096] | {g['fr'] / 1e9:.4f} GB | "
        f"{g['fw'] / 1e9:.4f} GB |\n"
        f"| k_bwd_large<4096, w FP32, gate, non-det> [{g['T']}, 4096] | {g['br'] / 1e9:.4f} GB | "
        f"{g['bw'] / 1e9:.4f} GB |" for g in gate)
    gate_table = "\n".join(
        f"| {g['T']} | {g['alg_f'] / 1e6:.1f} MB | {(g['fr'] + g['fw']) / 1e6:.1f} MB "
        f"({100 * ((g['fr'] + g['fw']) / g['alg_f'] - 1):+.2f}%) | {g['alg_b'] / 1e6:.1f} MB | "
        f"{(g['br'] + g['bw'] + fr + fw) / 1e6:.1f} MB "
        f"({100 * ((g['br'] + g['bw'] + fr + fw) / g['alg_b'] - 1):+.2f}%) | "
        f"{g['partials'] / 1e6:.1f} MB ({100 * g['partials'] / g['alg_b']:.1f}%) |" for g in gate)
    md = f"""# HBM traffic of the backward call at [131072, 4096] (rocprofv3 counters)

Commands (repository root $REPO, output directory $OUT, on an MI355X; committed files only; one counter per run):

```
cd /tmp && export TMPDIR=/tmp
timeout -s KILL 240 rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/pmc_fetch -o run -- python3 $REPO/bench.py --traffic-probe
timeout -s KILL 240 rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/pmc_write -o run -- python3 $REPO/bench.py --traffic-probe
python3 $REPO/bench.py --traffic-report $OUT/pmc_fetch $OUT/pmc_write <json> <this file>
```

`bench.py --traffic-probe` runs one 1 GiB device-to-device copy (torch `copy_`, dispatched as
`__amd_rocclr_copyBuffer`), the forward and the non-deterministic backward three times each at
[131072, 4096], then the gated forward and backward three times each at [16384, 4096],
[8192, 4096] and [3534, 4096] (dispatches told apart by their order).
Calibration with that copy of known size (1 GiB read, 1 GiB written): FETCH_SIZE read
{copy_kib(F):.1f} KiB and WRITE_SIZE {copy_kib(W):.1f} KiB, so read bytes = FETCH_SIZE x 1024 x
{ff:.5f} and written bytes = WRITE_SIZE x 1024 x {wf:.5f}.

| kernel (per dispatch, mean of 3) | read (scaled) | written (scaled) |
|---|---|---|
| k_bwd_large<4096, w FP32, plain, non-det> | {kr / 1e9:.4f} GB | {kw / 1e9:.4f} GB |
| k_fold | {fr / 1e9:.4f} GB | {fw / 1e6:.3f} MB |
| **backward call** | **{(kr + fr) / 1e9:.4f} GB** | **{(kw + fw) / 1e9:.4f} GB** |
| k_fwd<4096, w FP32, plain> [131072, 4096] | {fwr / 1e9:.4f} GB | {fww / 1e9:.4f} GB |
{gate_rows}

Algorithmic: reads x, dy, rstd, w = {(4 * T_HEAD * H_HEAD + 4 * T_HEAD + 4 * H_HEAD) / 1e9:.4f} GB;
writes dx, dw = {(2 * T_HEAD * H_HEAD + 4 * H_HEAD) / 1e9:.4f} GB; total {alg / 1e9:.4f} GB.
Measured {total / 1e9:.4f} GB per call, {100 * (total / alg - 1):.2f}% above it: the FP64 chunk
partials ({chunks} x {H_HEAD} x 8 B = {chunks * H_HEAD * 8 / 2**20:.0f} MiB) written by the main kernel and read back by the fold.
Forward at [131072, 4096]: algorithmic x read, y and rstd written, w read =
{alg_fwd / 1e9:.4f} GB; measured {(fwr + fww) / 1e9:.4f} GB ({100 * ((fwr + fww) / alg_fwd - 1):+.2f}%).
Gated form (forward: x, z read, y, rstd written, w; backward: x, dy, z, rstd, w read, dx, dz
written, dw), per call, the backward being main kernel + fold:

| gated [T, 4096] | fwd algorithmic | fwd measured | bwd algorithmic | bwd measured | FP64 partials written + read back |
|---|---|---|---|---|---|
{gate_table}

At the headline shape x, dy and dx are each moved once. Device sources hash: {out['kernel_hash']}
({", ".join(KERNEL_SOURCES)}); headline plan (path, chunks, sub-chains, fold group, grid, fold
grid, workspace bytes): {out['headline_plan']}. bench.py reports `traffic` only while both match
the current sources and plan.
"""
    with open(out_md, "w") as fh:
        fh.write(md)
    print(md)


def headline_setup():
    """Inputs of the headline workload on cuda:0, its forward's rstd and the
    backward workspace: (problem, x, dy, w, rstd, workspace, plan, y). The
    forward's y stays allocated for the caller, so the timed calls' dx lands
    where it always has relative to x and dy (placement moves this call)."""
    import torch

    import rmsnorm_train_fwd_amd as R
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating inputs [{T_HEAD}, {H_HEAD}]", file=sys.stderr, flush=True)
    p = synth.make(T_HEAD, H_HEAD, seed=0, w_dtype="f32")
    x = p.x.to(dev).view(T_HEAD, H_HEAD)
    dy = p.dy.to(dev).view(T_HEAD, H_HEAD)
    w = p.w.to(dev)
    y, rstd = R.rmsnorm_train_fwd(x, w, p.eps)
    plan_nd = R.rmsnorm_train_bwd_query(x, False)
    plan_d = R.rmsnorm_train_bwd_query(x, True)
    ws = torch.empty(max(plan_nd.workspace_bytes, plan_d.workspace_bytes), dtype=torch.uint8,
                     device=dev)
    torch.cuda.synchronize()
    return p, x, dy, w, rstd, ws, plan_nd, y


def run_to_run(band, ev):
    """Band of per-process medians: this process and the fresh ones."""
    meds = [round(ev[len(ev) // 2] * 1e3, 2)] + [b["median_us"] for b in band]
    lo, hi = min(meds), max(meds)
    nbytes = bwd_bytes(T_HEAD, H_HEAD, 4)
    return {"processes": len(meds), "median_us_per_process": meds, "band_us": [lo, hi],
            "band_frac_of_peak": [round(nbytes / (hi * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                                  round(nbytes / (lo * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)],
            "method": "median of the timed calls of each process (this one first, then fresh "
                      "processes started before this one used the GPU); value and frac use this "
                      "process's mean"}


def band_child(args):
    """One fresh process of the run-to-run band: the headline backward, K timed
    calls after W warm-up calls; prints its per-call median and mean (us)."""
    import torch

    import rmsnorm_train_fwd_amd as R

    p, x, dy, w, rstd, ws, _, y = headline_setup()
    ev, _ = time_calls(lambda: R.rmsnorm_train_bwd(dy, x, rstd, w, False, workspace=ws),
                       args.steps, args.warmup, torch)
    print(json.dumps({"median_us": round(ev[len(ev) // 2] * 1e3, 2),
                      "mean_us": round(sum(ev) / len(ev) * 1e3, 2)}), flush=True)


def run_band(args):
    """Per-process medians of the headline backward from args.band fresh
    processes (the pages take the median of the calls of each process and
    compare processes; where the caching allocator places x, dy and dx moves
    this call by several percent on MI355X)."""
    import subprocess

    out = []
    for i in range(args.band):
        print(f"[bench] run-to-run band: process {i + 1} of {args.band}", file=sys.stderr,
              flush=True)
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--band-child",
                            "--steps", str(args.steps), "--warmup", str(args.warmup)],
                           capture_output=True, text=True, timeout=600)
        if r.returncode != 0:
            raise SystemExit(f"bench.py: band process {i + 1} failed (exit {r.returncode}):\n"
                             f"{r.stderr[-2000:]}")
        out.append(json.loads(r.stdout.strip().splitlines()[-1]))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-rows", type=int, default=T_HEAD)
    ap.add_argument("--band", type=int, default=2,
                    help="fresh processes that repeat the headline timing for the run-to-run band")
    ap.add_argument("--band-child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--traffic-probe", action="store_true",
                    help="only run the copy + backward calls that the counter runs read")
    ap.add_argument("--sweep", metavar="OUT.md",
                    help="time every workload (cold caches, graph replay) into a markdown table")
    ap.add_argument("--sweep-kernels", nargs="+", metavar="ARG",
                    help="kernel-active times of a --sweep run traced by rocprofv3")
    ap.add_argument("--stats-report", nargs=2, metavar=("KERNEL_STATS.csv", "OUT.md"))
    ap.add_argument("--cpu-sweep", metavar="OUT.md",
                    help="time the FP64 CPU oracle on every workload (no GPU)")
    ap.add_argument("--traffic-report", nargs=4,
                    metavar=("FETCH_DIR", "WRITE_DIR", "OUT.json", "OUT.md"))
    args = ap.parse_args()
    if args.stats_report:
        stats_report(*args.stats_report,
                     "rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/prof_bench "
                     "-o run -- python3 $REPO/bench.py")
        return
    if args.traffic_report:
        traffic_report(*args.traffic_report)
        return
    if args.cpu_sweep:
        cpu_sweep(args.cpu_sweep)
        return
    if args.sweep_kernels:
        sweep_kernels(args.sweep_kernels[:-1], args.sweep_kernels[-1])
        return
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU only; --gpus {args.gpus} is not supported "
              "(rows shard across GPUs with no exchange for the forward and dx and one "
              "exchange of the FP64 dw per backward call; only one GPU is measured here)",
              file=sys.stderr)
        sys.exit(2)

    if args.traffic_probe:
        traffic_probe()
        return
    if args.sweep:
        sweep(args.sweep)
        return

    if args.band_child:
        band_child(args)
        return
    # Fresh processes first, before this one touches the GPU: each times the
    # same backward on its own allocation of the same inputs. Under a profiler
    # (its library preloaded) the GPU is initialised before this program
    # starts, so no child process is started from it and the band is skipped.
    profiled = "rocprof" in os.environ.get("LD_PRELOAD", "")
    if profiled and args.band > 0:
        print("[bench] run-to-run band skipped: running under a profiler", file=sys.stderr,
              flush=True)
    band = run_band(args) if args.band > 0 and not profiled else []

    import torch

    import rmsnorm_train_fwd_amd as R

    p, x, dy, w, rstd, ws, plan_nd, y = headline_setup()

    def bwd_nd():
        R.rmsnorm_train_bwd(dy, x, rstd, w, False, workspace=ws)

    def bwd_d():
        R.rmsnorm_train_bwd(dy, x, rstd, w, True, workspace=ws)

    def fwd():
        R.rmsnorm_train_fwd(x, w, p.eps)

    print("[bench] timing backward (non-deterministic)", file=sys.stderr, flush=True)
    ev, wall = time_calls(bwd_nd, args.steps, args.warmup, torch)
    print("[bench] timing backward (deterministic) and forward", file=sys.stderr, flush=True)
    ev_d, _ = time_calls(bwd_d, max(10, args.steps // 2), 3, torch)
    ev_f, _ = time_calls(fwd, max(10, args.steps // 2), 3, torch)
    print("[bench] timing the bandwidth probe", file=sys.stderr, flush=True)
    ceiling = stream_ceiling(x, dy, max(10, args.steps // 2), torch)

    def med(v):
        return v[len(v) // 2]

    mean_ms = sum(ev) / len(ev)
    nbytes = bwd_bytes(T_HEAD, H_HEAD, 4)
    gbps = nbytes / (mean_ms * 1e-3) / 1e9
    traffic = measured_traffic()
    result = {
        "metric": "bwd us/call and achieved HBM GB/s (% of peak) at [131072,4096] BF16",
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(gbps / (nbytes / (PAGES_BWD_US_B200 * 1e-6) / 1e9), 4),
        "dtype": "f32",
        "data": "synthetic: x, dy ~ N(0,1) cast to BF16, w = 1 + 0.1 N(0,1) FP32, seed 0",
        "config": {
            "workload": "rmsnorm_train_bwd non-deterministic, x/dy/dx BF16 [131072, 4096], "
                        "w FP32, dw FP32, eps 1e-6",
            "T": T_HEAD, "H": H_HEAD, "w_dtype": "f32", "deterministic": False,
            "algorithmic_bytes_per_call": nbytes,
            "workspace_bytes": plan_nd.workspace_bytes,
        },
        "us_per_call": {"mean": round(mean_ms * 1e3, 2), "median": round(med(ev) * 1e3, 2),
                        "p10": round(ev[len(ev) // 10] * 1e3, 2),
                        "p90": round(ev[(9 * len(ev)) // 10] * 1e3, 2)},
        "roofline": {
            "bound": "hbm",
            "kernel": "backward call: k_bwd_large + k_fold (HIP events around each call)",
            "achieved": round(gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
        },
        "extra": {
            "bwd_det_us": round(med(ev_d) * 1e3, 2),
            "bwd_det_GBps": round(bwd_bytes(T_HEAD, H_HEAD, 4) / (med(ev_d) * 1e-3) / 1e9, 1),
            "fwd_us": round(med(ev_f) * 1e3, 2),
            "fwd_GBps": round(fwd_bytes(T_HEAD, H_HEAD, 4) / (med(ev_f) * 1e-3) / 1e9, 1),
            "ceiling": ceiling,
            "bwd_vs_r2w1_ceiling": round(gbps / ceiling["r2w1_GBps"], 4) if ceiling else None,
            "run_to_run": run_to_run(band, ev),
            "baseline": {"us_per_call": PAGES_BWD_US_B200,
                         "GBps": round(nbytes / (PAGES_BWD_US_B200 * 1e-6) / 1e9, 1),
                         "hardware": "NVIDIA B200 (sm_100a)",
                         "source": "the pages' non-deterministic backward at this workload; "
                                   "another machine's number: context, not the target"},
        },
    }
    if not args.no_cpu:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(p, args.cpu_rows)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
