#!/usr/bin/env python3
"""Throughput of ragged paged attention on one MI355X.

    python bench.py [--workload decode] [--steps K] [--warmup W] [--gpus 1]

A step is one ``rpa_forward`` call over one batch of seeded synthetic input
(bf16 N(0,1) Q/K/V, shuffled page tables) already resident in HBM.  The
default workload is the decode batch: 128 single-token sequences with kv_len
~ U[64, 640], 8 query heads sharing one KV head of width 256, 128-token pages.

So that no step finds its inputs in the 256 MB last-level cache, the bench
keeps R replicas of the inputs (at least 1 GiB in total, at most 64 of them:
a workload of a few KB stays cache resident) and step i reads replica i mod R.  The library's kernel timing (HIP events recorded on the
launch stream directly around every kernel) gives each kernel's duration
behind ``roofline.achieved``; the wall clock over the K timed steps gives
``value`` and ``ms_per_step``.  The oracle's CPU time on a bounded sample of
the same workload is reported as ``cpu_baseline``.

``--append`` makes every step call ``rpa_forward_append`` instead: the step's
new K/V rows are written into their pages (the same bytes each step) before the
attention kernels, and the append kernel is timed beside them.

``--kv fp8`` holds the K/V pools as OCP FP8 E4M3 bytes with per-KV-head scales
(drawn from the same bf16 values) and calls ``rpa_forward_fp8`` (with
``--append``: ``rpa_forward_fp8_append``, which quantizes the new rows); the
K/V bytes of the roofline are then one byte per element.

By default the same run also times the other workloads of the metric (the
8192-token window-1024 and global prefills, the tiny prefill and the two mixed
chunked-prefill steps) and reports each under ``configs``, with its dominant
kernel's duration and roofline fraction (``--configs ''`` skips them).
``--stack`` adds one step of a 5 window-1024 : 1 global layer stack, timed
eagerly and as one captured HIP graph.

Prints ONE JSON line.

Counter runs (HBM traffic of the dominant kernel):

    rocprofv3 --pmc FETCH_SIZE -d DIR_F -o run -- python3 bench.py --steps 8 --warmup 2 \
        --no-cpu-baseline --copy-calibration
    rocprofv3 --pmc WRITE_SIZE -d DIR_W -o run -- python3 bench.py ...same...
    python3 bench.py --pmc-summary DIR_F DIR_W      # writes profiles/traffic_<workload>.json

The copy calibration runs a plain elementwise kernel over a buffer of known
size in the same process, so that the counters can be scaled to bytes.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention tokens/s + achieved TFLOP/s (prefill) and KV GB/s (decode), % of peak"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
LLC_BYTES = 256 << 20
CSRC = os.path.join(ROOT, "ragged_paged_attention_forward_amd", "csrc")
COPY_BYTES = 1 << 30            # calibration buffer (read once, written once)
KERNEL_NAMES = {"prefill": "rpa_prefill_kernel", "decode": "rpa_decode_kernel", "merge": "rpa_merge_kernel",
                "append": "rpa_append_kernel", "stage": "rpa_stage_kernel", "decode2": "rpa_decode_kernel"}
WORKLOADS = ("decode", "tiny", "swa_prefill", "global_prefill", "mixed", "mixed_swa", "swa_prefill_share8",
             "global_prefill_share2")
# read-probe shapes swept for the measured HBM ceiling: (workgroups, threads,
# 16-byte loads in flight per thread), from one workgroup per compute unit
# with deep queues to many small workgroups
PROBE_SHAPES = [(256, 1024, 8), (256, 1024, 16), (256, 256, 32), (512, 256, 16), (512, 1024, 4),
                (1024, 256, 8), (1024, 256, 16), (2048, 256, 4), (2048, 256, 8), (4096, 256, 4),
                (8192, 256, 4), (1024, 1024, 4)]


def kernel_source_hash() -> str:
    """Hash of every kernel and host source of the library."""
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(CSRC, "*"))):
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, kernel: str, kv: str = "bf16"):
    """HBM bytes per launch from committed rocprofv3 counter runs, if still current."""
    tag = workload if kv == "bf16" else f"{workload}_{kv}"
    path = os.path.join(ROOT, "profiles", f"traffic_{tag}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash() or rec.get("kernel") != kernel:
        return None
    return rec.get("hbm_bytes_per_launch")


def kernel_work(w, items, merge_kernel=True, kv_elem_bytes=2):
    """Algorithmic FLOPs and bytes of each kernel kind for the planned step.

    A sequence belongs to the kernel kind of its work items.  Bytes count Q,
    the unique K/V rows its queries see and its page-table entries; O goes to
    the kernel that writes it (the merge kernel for split sequences when it
    runs, else the prefill or decode kernel, whose last split merges them).
    """
    from ragged_paged_attention_forward_amd import metrics
    kind_of = {}
    split = set()
    for it in items:
        kind_of[it["seq"]] = {1: "decode", 2: "decode2"}.get(it["kind"], "prefill")
        if it["num_splits"] > 1:
            split.add(it["seq"])
    out = {}
    for kind in ("prefill", "decode", "decode2"):
        ids = [s for s, k in kind_of.items() if k == kind]
        seqs = [w.seqs[s] for s in ids]
        q_b = metrics.qo_bytes(seqs, w.num_q_heads, w.head_dim) // 2
        o_ids = ids if not merge_kernel else [s for s in ids if s not in split]
        o_b = metrics.qo_bytes([w.seqs[s] for s in o_ids], w.num_q_heads, w.head_dim) // 2
        kv = metrics.kv_bytes(seqs, w.window, w.num_kv_heads, w.head_dim) * kv_elem_bytes // 2
        pages = sum(-(-kvl // w.page_size) for _, kvl in seqs) * 4
        out[kind] = {"flops": int(metrics.flops(seqs, w.window, w.num_q_heads, w.head_dim)),
                     "bytes": int(q_b + o_b + kv + pages), "seqs": len(seqs)}
    # the merge writes O of the split sequences (its fp32 partial reads are overhead)
    seqs = [w.seqs[s] for s in sorted(split)]
    out["merge"] = {"flops": 0, "bytes": int(metrics.qo_bytes(seqs, w.num_q_heads, w.head_dim) // 2),
                    "seqs": len(seqs)}
    # the KV append reads the step's new K and V rows and writes them into their pages
    new_elems = w.total_q * w.num_kv_heads * w.head_dim * 2   # K and V
    out["append"] = {"flops": 0, "bytes": int(new_elems * (2 + kv_elem_bytes)), "seqs": w.num_seqs}
    # fp8 staging: the prefill sequences' pages read as bytes, written as bf16
    pre = [w.seqs[s] for s, k in kind_of.items() if k == "prefill"]
    staged = sum(-(-kvl // w.page_size) for _, kvl in pre) * w.page_size * w.num_kv_heads * w.head_dim * 2
    out["stage"] = {"flops": 0, "bytes": int(3 * staged), "seqs": len(pre)}
    return out


def new_row_slots(w, cu, kv, page_table) -> np.ndarray:
    """Flat page-slot index (page * page_size + slot) of each of the step's new
    tokens, in token order: token r of sequence s is at position
    kv_len - q_len + r (bench input construction for the append mode)."""
    b = w.page_size
    out = []
    for s in range(w.num_seqs):
        pos = np.arange(int(kv[s]) - int(cu[s + 1] - cu[s]), int(kv[s]))
        out.append(page_table[s][pos // b].astype(np.int64) * b + pos % b)
    return np.concatenate(out) if out else np.zeros(0, dtype=np.int64)


def cpu_baseline(w, budget_s: float):
    """Time the fp64 oracle on a bounded sample of the workload on the host cores."""
    import oracle.rpa_oracle as ora
    import rpa_workloads as wl
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    host_cores = len(os.sched_getaffinity(0))
    cores = min(host_cores, max(1, blas_threads))   # threads the oracle's BLAS products use
    inp = wl.make_inputs(w)
    cu = inp.cu_q_lens.tolist()
    t_total = cu[-1]
    # sample: whole sequences for short ones, a random set of rows for long
    # prefills; passes over the batch repeat until the time budget is spent
    rng = np.random.default_rng(w.seed)
    done_tokens = 0
    rows_per_call = 64
    n_seq = 0
    passes = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        passes += 1
        for s in rng.permutation(w.num_seqs):
            q_len = cu[s + 1] - cu[s]
            if q_len == 0:
                continue
            if q_len <= rows_per_call:
                rows = list(range(cu[s], cu[s + 1]))
            else:
                rows = sorted(rng.choice(np.arange(cu[s], cu[s + 1]), rows_per_call, replace=False).tolist())
            ora.forward_rows(inp.q, inp.k_pages, inp.v_pages, inp.page_table, inp.cu_q_lens,
                             inp.kv_lens, inp.window, inp.scale, rows)
            done_tokens += len(rows)
            n_seq += 1
            if time.perf_counter() - t0 > budget_s:
                break
    el = time.perf_counter() - t0
    return {"value": round(done_tokens / el, 2), "unit": "tokens/s", "cores": int(cores),
            "host_cores": int(host_cores), "blas_threads": int(blas_threads), "kind": "oracle",
            "sample": f"{done_tokens} query tokens of a {t_total}-token step ({n_seq} sequence "
                      f"visits over {passes} pass(es), up to {rows_per_call} rows each, fp64 numpy) "
                      f"in {el:.1f} s",
            "seconds": round(el, 2)}


def stats_ms(a):
    a = np.asarray(a, dtype=np.float64)
    if a.size == 0:
        return None
    return {"launches": int(a.size), "mean_ms": round(float(a.mean()), 6),
            "p10_ms": round(float(np.percentile(a, 10)), 6), "p50_ms": round(float(np.median(a)), 6),
            "p90_ms": round(float(np.percentile(a, 90)), 6)}


_SLEEP_CAL = []


def sleep_cycles_per_ms(torch) -> float:
    """Cycles of torch.cuda._sleep per millisecond, measured once with events."""
    if not _SLEEP_CAL:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        a.record()
        torch.cuda._sleep(20_000_000)
        b.record()
        torch.cuda.synchronize()
        _SLEEP_CAL.append(20_000_000 / max(a.elapsed_time(b), 1e-3))
    return _SLEEP_CAL[0]


def copy_calibration(torch, dev):
    """A plain elementwise kernel over COPY_BYTES: reads them once and writes them once."""
    a = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    del a, b


def measured_peak(torch, R, dev, bound: str, nbytes: int):
    """What the device sustains for the dominant kernel's bound, measured here:
    a plain streaming read of the same byte count from cold memory (best of
    two grid sizes), or independent bf16 MFMA chains on every compute unit."""
    stream = torch.cuda.current_stream(dev)

    def time_launches(launch, n):
        ts = []
        for i in range(n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch(i)
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    if bound == "hbm":
        nb = max(16, (int(nbytes) + 15) // 16 * 16)
        slices = max(4, int(np.ceil(4 * LLC_BYTES / nb)))   # rotate so no read finds its slice in the LLC
        pool = torch.empty(nb * slices, dtype=torch.uint8, device=dev)
        pool.fill_(1)
        best, best_shape, sweep = None, None, {}
        for wgs, threads, loads in PROBE_SHAPES:
            sink = torch.empty(wgs * threads, dtype=torch.int32, device=dev)
            launch = lambda i: R.probe_read(pool[(i % slices) * nb:], nb, wgs, sink, stream, threads, loads)
            time_launches(launch, 3)
            ms = time_launches(launch, 25)
            sweep[f"{wgs}x{threads}x{loads}"] = round(nb / (ms * 1e-3) / 1e9, 1)
            if best is None or ms < best:
                best, best_shape = ms, (wgs, threads, loads)
        del pool
        return {"value": round(nb / (best * 1e-3) / 1e9, 1), "unit": "GB/s",
                "probe": f"rpa_probe_read: plain streaming read of the same {nb} bytes, cold "
                         f"(rotated over {slices} slices), median of 25 launches per shape, best of "
                         f"{len(PROBE_SHAPES)} shapes (workgroups x threads x 16-byte loads in flight per "
                         f"thread): {best_shape[0]}x{best_shape[1]}x{best_shape[2]}",
                "sweep_gbps": sweep}
    wgs, iters = 1024, 2048
    sink = torch.empty(wgs * 512, dtype=torch.float32, device=dev)
    flops = R.probe_mfma(wgs, iters, sink, stream)
    launch = lambda i: R.probe_mfma(wgs, iters, sink, stream)
    time_launches(launch, 2)
    ms = time_launches(launch, 5)
    return {"value": round(flops / (ms * 1e-3) / 1e12, 1), "unit": "TFLOP/s",
            "probe": f"rpa_probe_mfma: {wgs} workgroups x 8 waves x {iters} x 4 independent "
                     "v_mfma_f32_32x32x16_bf16, median of 5 launches"}


def graph_layers(torch, attn, replicas, w, cu, kv, layers: int, stream):
    """The attention calls of `layers` layers of one step (same metadata, one
    input replica per layer) launched eagerly and replayed as one captured HIP
    graph: wall time per layer of each."""
    n = min(layers, len(replicas))
    outs = [torch.empty_like(replicas[i][0].q) for i in range(n)]

    def calls():
        for i in range(n):
            d = replicas[i][0]
            attn.forward(d.q, d.k_pages, d.v_pages, d.page_table, cu, kv, w.window, w.scale, out=outs[i])

    calls()                      # the work list is on the device before the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    reps = max(20, 2000 // n)

    def timed(fn):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / reps / n * 1e3

    def eager():
        with torch.cuda.stream(stream):
            calls()
    eager_ms = timed(eager)
    graph_ms = timed(g.replay)
    return {"layers": n, "eager_ms_per_layer": round(eager_ms, 6), "graph_ms_per_layer": round(graph_ms, 6),
            "replays": reps}


def library_options(args):
    """(name, value) pairs of --set NAME=VALUE (RPA_OPT_<NAME> of the library)."""
    out = []
    for item in args.set or []:
        name, _, value = item.partition("=")
        out.append((name.strip().upper(), int(value)))
    return out


def measure(args, workload: str, torch, R, dev, graph_layers_n: int = 0):
    """Time one workload: K wall-clock steps (``value``, ``ms_per_step``), then
    the event-timed pass for each kernel's duration and the roofline of the
    dominant kernel.  Returns the result dict (without the CPU baseline)."""
    import rpa_workloads as wl

    w = wl.by_name(workload)
    fp8 = args.kv == "fp8"
    if fp8:
        host8 = wl.make_fp8_inputs(w)
        host = host8.base
        k16, v16 = host.k_pages, host.v_pages                      # bf16 rows the fp8 append writes
        host.k_pages, host.v_pages = host8.k_pages, host8.v_pages   # the pools the steps read
    else:
        host = wl.make_inputs(w)
    t_q = w.total_q
    per_replica = sum(t.numel() * t.element_size() for t in (host.q, host.k_pages, host.v_pages)) * 2
    # enough replicas that the set exceeds the last-level cache four times,
    # at most 64 (small workloads then stay cache resident, like in serving)
    reps = args.replicas or min(64, max(2, int(np.ceil(4 * LLC_BYTES / per_replica))))
    replicas = []
    for _ in range(reps):
        d = host.to(dev)
        replicas.append((d, torch.empty_like(d.q)))
    if fp8:
        k_scales, v_scales = host8.k_scales.to(dev), host8.v_scales.to(dev)
    cu = np.ascontiguousarray(host.cu_q_lens.numpy().astype(np.int32))
    kv = np.ascontiguousarray(host.kv_lens.numpy().astype(np.int32))

    attn = R.RaggedPagedAttention(w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size,
                                  w.num_seqs, w.max_pages_per_seq, t_q)
    for name, value in library_options(args):
        attn.set_option(getattr(R, "RPA_OPT_" + name), value)
    info, items = attn.plan(cu, kv, w.window)
    # host metadata builder: one rpa_plan call (work list built, not copied out), best of 20
    plan_s = []
    for _ in range(20):
        t_plan = time.perf_counter()
        attn.plan_info(cu, kv, w.window)
        plan_s.append(time.perf_counter() - t_plan)
    planner_us = min(plan_s) * 1e6
    stream = torch.cuda.current_stream(dev)

    if args.append:
        # each step also writes its new K/V rows (already in the pages, so every
        # step writes the same bytes) through rpa_forward_append
        slots = torch.from_numpy(new_row_slots(w, cu, kv, host.page_table.numpy())).to(dev)
        news = []
        flat = (w.num_kv_heads, w.head_dim)
        for d, _ in replicas:
            if fp8:   # the bf16 rows whose quantized bytes the pools already hold
                news.append((k16.reshape(-1, *flat)[slots.cpu()].contiguous().to(dev),
                             v16.reshape(-1, *flat)[slots.cpu()].contiguous().to(dev)))
            else:
                news.append((d.k_pages.view(-1, *flat)[slots].contiguous(),
                             d.v_pages.view(-1, *flat)[slots].contiguous()))

    def step(i):
        d, out = replicas[i % reps]
        if args.append and fp8:
            kn, vn = news[i % reps]
            attn.forward_fp8_append(d.q, kn, vn, d.k_pages, d.v_pages, k_scales, v_scales, d.page_table, cu, kv,
                                    w.window, w.scale, out=out, stream=stream)
            return
        if args.append:
            kn, vn = news[i % reps]
            attn.forward_append(d.q, kn, vn, d.k_pages, d.v_pages, d.page_table, cu, kv, w.window, w.scale,
                                out=out, stream=stream)
            return
        if fp8:
            attn.forward_fp8(d.q, d.k_pages, d.v_pages, k_scales, v_scales, d.page_table, cu, kv, w.window,
                             w.scale, out=out, stream=stream)
            return
        attn.forward(d.q, d.k_pages, d.v_pages, d.page_table, cu, kv, w.window, w.scale, out=out,
                     stream=stream)

    torch.cuda.synchronize()
    t_cold = time.perf_counter()
    step(0)   # builds the plan and uploads the work list
    torch.cuda.synchronize()
    cold_ms = (time.perf_counter() - t_cold) * 1e3
    for i in range(args.warmup):
        step(1 + i)
    torch.cuda.synchronize()

    # Timed region: K steps, wall clock, no instrumentation.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(1 + args.warmup + i)
    t_enq = time.perf_counter()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    enqueue_ms = (t_enq - t0) * 1e3 / args.steps

    # Kernel durations: up to --timing-steps of the same steps again with the library's HIP events
    # around every kernel.  A sleep kernel queued first lets the host run
    # ahead, so that no kernel waits for its own launch inside its brackets;
    # untimed steps between the sleep and the timed ones bring the device
    # back to the clock it holds under the steady load of the timed region.
    timed = min(args.steps, args.timing_steps)
    settle = max(4, int(np.ceil(2.0 / max(wall * 1e3 / args.steps, 1e-3))))   # about 2 ms of steps
    head_ms = 1.5 * enqueue_ms * (timed + settle) + 1.0
    torch.cuda.synchronize()
    torch.cuda._sleep(int(head_ms * sleep_cycles_per_ms(torch)))
    for i in range(settle):
        step(1 + args.warmup + args.steps + i)
    attn.set_option(R.RPA_OPT_KERNEL_TIMING, timed)
    for i in range(timed):
        step(1 + args.warmup + args.steps + settle + i)
    torch.cuda.synchronize()
    kernels = {}
    for name, kind in R.KERNEL_KINDS.items():
        st = stats_ms(attn.kernel_times(kind))
        if st is not None:
            kernels[name] = st
    attn.set_option(R.RPA_OPT_KERNEL_TIMING, 0)

    kv_elem = 1 if fp8 else 2
    work = kernel_work(w, items, merge_kernel="merge" in kernels, kv_elem_bytes=kv_elem)
    # The dominant kernel is the one with the largest roofline time (its
    # algorithmic FLOPs at the MFMA peak or bytes at the HBM peak, whichever
    # is larger): with the decode kernel on a second stream, durations overlap
    # and the longest one need not be the one that bounds the step.
    def roof_s(k):
        return max(work[k]["flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12), work[k]["bytes"] / (HBM_PEAK_GBS * 1e9))
    dom = max(kernels, key=roof_s)
    kw = work[dom]
    k_ms = kernels[dom]["mean_ms"]
    t_mfma = kw["flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    t_hbm = kw["bytes"] / (HBM_PEAK_GBS * 1e9)
    if t_mfma >= t_hbm:
        bound, achieved, peak, unit = "mfma", kw["flops"] / (k_ms * 1e-3) / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    else:
        bound, achieved, peak, unit = "hbm", kw["bytes"] / (k_ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"
    mp = measured_peak(torch, R, dev, bound, kw["bytes"])
    mp["frac"] = round(achieved / mp["value"], 4)
    roofline = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "measured_peak": mp,
                "traffic": load_traffic(workload, KERNEL_NAMES[dom], args.kv),
                "kernel": KERNEL_NAMES[dom], "kernel_ms_mean": k_ms,
                "algorithmic_bytes": kw["bytes"], "algorithmic_flops": kw["flops"],
                "source_sha256_16": kernel_source_hash()}

    from ragged_paged_attention_forward_amd import metrics
    step_flops = metrics.flops(w.seqs, w.window, w.num_q_heads, w.head_dim)
    kv_b = metrics.kv_bytes(w.seqs, w.window, w.num_kv_heads, w.head_dim) * kv_elem // 2
    step_bytes = metrics.total_bytes(w.seqs, w.window, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                     w.page_size) - metrics.kv_bytes(w.seqs, w.window, w.num_kv_heads,
                                                                     w.head_dim) + kv_b
    assert info["visible_pairs"] == metrics.visible_pairs(w.seqs, w.window)
    ms_per_step = wall * 1e3 / args.steps
    for name in kernels:
        kernels[name]["algorithmic_bytes"] = work[name]["bytes"]
        kernels[name]["algorithmic_flops"] = work[name]["flops"]

    res = {
        "metric": METRIC,
        "value": round(t_q * args.steps / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V, shuffled page tables)",
        "config": {"workload": workload, "description": w.description, "seed": w.seed,
                   "num_seqs": w.num_seqs, "q_tokens": t_q, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "page_size": w.page_size, "window": w.window, "replicas": reps, "append_kv": bool(args.append),
                   "kv_dtype": "fp8_e4m3" if fp8 else "bf16",
                   "options": {n: v for n, v in library_options(args)},
                   "parallelism": "single GPU"},
        "step_tflops": round(step_flops / (ms_per_step * 1e-3) / 1e12, 3),
        "step_hbm_gbps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "step_kv_gbps": round(kv_b / (ms_per_step * 1e-3) / 1e9, 1),
        "enqueue_ms_per_step": round(enqueue_ms, 6),
        "planner_us": round(planner_us, 1),
        "cold_call_ms": round(cold_ms, 3),
        "kernels": kernels,
        "plan": info,
        "roofline": roofline,
    }
    if graph_layers_n > 0:
        res["graph"] = graph_layers(torch, attn, replicas, w, cu, kv, graph_layers_n, stream)
    if args.stack:
        res["stack"] = layer_stack(torch, attn, replicas, w, cu, kv, stream)
    attn.close()
    del replicas
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def table_sweep(args, torch, R, dev):
    """One call per entry of the planner's (head size, group, regime, cache)
    table: 64 sequences of q_len tokens (1: decode; 2 and 4: few-token
    steps; 16: a short chunk) with keys U[64, 768] per entry, plus one
    2048-token prefill per head size; each entry's kernels and their mean
    duration over a few calls (library events).  Run under rocprofv3, the
    kernel trace names every entry's kernel instantiation."""
    import rpa_workloads as wl
    rows = []
    for d in (64, 128, 256, 512):
        for g in (1, 2, 4, 8, 16, 32):
            for q in (1, 2, 4, 16):
                for kv8 in (False, True):
                    rng = np.random.default_rng(d + g + q)
                    w = wl.custom([(q, int(k)) for k in rng.integers(64 + q, 769, 64)], g, 1, d, 128, 0, seed=7)
                    rows.append(_table_entry(torch, R, dev, w, kv8, f"d{d} G{g} q{q} {'fp8' if kv8 else 'bf16'}"))
        w = wl.custom([(2048, 2048)], 8, 1, d, 128, 0, seed=8)
        for kv8 in (False, True):
            rows.append(_table_entry(torch, R, dev, w, kv8, f"d{d} G8 q2048 {'fp8' if kv8 else 'bf16'}"))
    return rows


TABLE_DECODE_ROWS = [0]   # --decode-max-rows for the table sweep (0: the library's table)


def _table_entry(torch, R, dev, w, kv8, label):
    import rpa_workloads as wl
    if kv8:
        f = wl.make_fp8_inputs(w).to(dev)
        d, host = f.base, f.base
    else:
        d = host = wl.make_inputs(w).to(dev)
    attn = R.RaggedPagedAttention(w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size, w.num_seqs,
                                  w.max_pages_per_seq, w.total_q)
    if TABLE_DECODE_ROWS[0]:
        attn.set_option(R.RPA_OPT_DECODE_MAX_ROWS, TABLE_DECODE_ROWS[0])
    out = torch.empty_like(d.q)

    def call():
        if kv8:
            attn.forward_fp8(d.q, f.k_pages, f.v_pages, f.k_scales, f.v_scales, d.page_table, host.cu_q_lens,
                             host.kv_lens, 0, w.scale, out=out)
        else:
            attn.forward(d.q, d.k_pages, d.v_pages, d.page_table, host.cu_q_lens, host.kv_lens, 0, w.scale, out=out)
    call()
    torch.cuda.synchronize()
    attn.set_option(R.RPA_OPT_KERNEL_TIMING, 5)
    for _ in range(5):
        call()
    torch.cuda.synchronize()
    ks = {}
    for name, kind in R.KERNEL_KINDS.items():
        t = attn.kernel_times(kind)
        if len(t):
            ks[name] = round(float(np.mean(t)) * 1e3, 2)
    attn.close()
    return {"entry": label, "kernels_us": ks}


def config_summary(res):
    """The fields of one workload's result that the `configs` record keeps."""
    r = res["roofline"]
    return {"workload": res["config"]["workload"], "description": res["config"]["description"],
            "value": res["value"], "unit": res["unit"], "ms_per_step": res["ms_per_step"],
            "kernels": {k: {"mean_ms": v["mean_ms"], "p50_ms": v["p50_ms"]} for k, v in res["kernels"].items()},
            "roofline": {k: r[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic", "kernel",
                                          "kernel_ms_mean", "algorithmic_bytes", "algorithmic_flops")},
            "measured_peak": {"value": r["measured_peak"]["value"], "unit": r["measured_peak"]["unit"],
                              "frac": r["measured_peak"]["frac"]},
            "step_tflops": res["step_tflops"], "step_kv_gbps": res["step_kv_gbps"],
            "enqueue_ms_per_step": res["enqueue_ms_per_step"], "plan": res["plan"]}


def layer_stack(torch, attn, replicas, w, cu, kv, stream, pattern=(1024, 1024, 1024, 1024, 1024, 0)):
    """One step of a layer stack of five sliding-window layers and one global
    layer (the pages' 5:1 pattern) on the workload's metadata: six calls, each
    on its own input replica, two work lists (one per window).  Timed as eager
    calls and as one captured HIP graph replayed; wall time per step."""
    n = len(pattern)
    outs = [torch.empty_like(replicas[i % len(replicas)][0].q) for i in range(n)]

    def calls():
        for i, win in enumerate(pattern):
            d = replicas[i % len(replicas)][0]
            attn.forward(d.q, d.k_pages, d.v_pages, d.page_table, cu, kv, win, w.scale, out=outs[i])

    calls()                      # both work lists are on the device before the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    reps = 50

    def timed(fn):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / reps * 1e3

    def eager():
        with torch.cuda.stream(stream):
            calls()
    eager_ms = timed(eager)
    graph_ms = timed(g.replay)
    attn.release_captured()
    return {"pattern": list(pattern), "eager_ms_per_step": round(eager_ms, 6),
            "graph_ms_per_step": round(graph_ms, 6), "replays": reps,
            "tokens_per_s_graph": round(w.total_q * n / (graph_ms * 1e-3), 1)}


def run(args):
    import torch
    import ragged_paged_attention_forward_amd as R

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.table:
        TABLE_DECODE_ROWS[0] = args.decode_max_rows
        rows = table_sweep(args, torch, R, dev)
        print(json.dumps({"table": rows}), flush=True)
        return 0
    res = measure(args, args.workload, torch, R, dev, args.graph_layers)
    if args.configs:
        # the other workloads of the metric (the prefill half: TFLOP/s of the
        # 8192-token prefills; the mixed steps), each timed the same way
        others = [x for x in (args.configs.split(",") if args.configs != "all" else WORKLOADS)
                  if x != args.workload]
        res["configs"] = {}
        for name in others:
            print(f"# measuring {name}", file=sys.stderr, flush=True)
            res["configs"][name] = config_summary(measure(args, name, torch, R, dev))
    if args.copy_calibration:
        copy_calibration(torch, dev)
    if not args.no_cpu_baseline and args.kv != "fp8":
        import rpa_workloads as wl
        res["cpu_baseline"] = cpu_baseline(wl.by_name(args.workload), args.cpu_budget)
    print(json.dumps(res), flush=True)
    return 0


def _pmc_per_dispatch(d, counter):
    """Per-dispatch values of one counter for every kernel name in a rocprofv3 output dir."""
    import sqlite3
    dbs = sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True))
    if not dbs:
        raise SystemExit(f"no rocprofv3 database under {d}")
    vals = {}
    for db in dbs:
        con = sqlite3.connect(db)
        cols = [r[1] for r in con.execute("pragma table_info(pmc_events)")]
        key = "dispatch_id" if "dispatch_id" in cols else "rowid"
        q = (f"select name, {key}, sum(counter_value) from pmc_events where counter_name = ? "
             f"group by name, {key}")
        for name, _, v in con.execute(q, (counter,)):
            vals.setdefault(name, []).append(float(v))
        con.close()
    return vals


def trace_summary(args):
    """Markdown kernel statistics (calls, mean / min / max duration, share)
    from a rocprofv3 --kernel-trace database (the `kernels` view of its rocpd
    file)."""
    import sqlite3
    dbs = sorted(glob.glob(os.path.join(args.trace_summary, "**", "*.db"), recursive=True))
    if not dbs:
        raise SystemExit(f"no rocprofv3 database under {args.trace_summary}")
    stats = {}
    for db in dbs:
        con = sqlite3.connect(db)
        for name, dur in con.execute("select name, duration from kernels"):
            stats.setdefault(name, []).append(dur / 1e3)
        con.close()
    total = sum(sum(v) for v in stats.values())
    lines = ["| kernel | calls | average (us) | min (us) | max (us) | share |",
             "|---|---|---|---|---|---|"]
    for name, v in sorted(stats.items(), key=lambda kv: -sum(kv[1])):
        a = np.asarray(v)
        short = name.split("(")[0] if name.startswith("void rpa::") else name
        lines.append(f"| `{short}` | {a.size} | {a.mean():.2f} | {a.min():.2f} | {a.max():.2f} | "
                     f"{100 * a.sum() / total:.1f} % |")
    print("\n".join(lines))
    return 0


def pmc_summary(args):
    """Turn a FETCH_SIZE and a WRITE_SIZE run into HBM bytes per launch of the dominant kernel."""
    fdir, wdir = args.pmc_summary
    fetch = _pmc_per_dispatch(fdir, "FETCH_SIZE")
    write = _pmc_per_dispatch(wdir, "WRITE_SIZE")

    def pick(vals, needle):
        names = [n for n in vals if needle in n]
        if not names:
            raise SystemExit(f"no dispatch of {needle} in the counter run")
        v = [x for n in names for x in vals[n]]
        return float(np.mean(v)), len(v)

    cf, _ = pick(fetch, "neg")        # KiB per dispatch of the calibration kernel
    cw, _ = pick(write, "neg")
    f_scale = COPY_BYTES / (cf * 1024.0)
    w_scale = COPY_BYTES / (cw * 1024.0)
    kernel = args.pmc_kernel
    kf, nf = pick(fetch, kernel)
    kwr, nw = pick(write, kernel)
    rec = {
        "workload": args.workload, "kv_dtype": args.kv, "kernel": kernel,
        "kernel_source_sha256_16": kernel_source_hash(),
        "fetch_kib_per_dispatch": round(kf, 1), "write_kib_per_dispatch": round(kwr, 1),
        "dispatches": [nf, nw],
        "calibration": {"kernel": "torch.neg over a bf16 buffer", "bytes": COPY_BYTES,
                        "fetch_kib": round(cf, 1), "write_kib": round(cw, 1),
                        "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)},
        "hbm_bytes_per_launch": int(round(kf * 1024.0 * f_scale + kwr * 1024.0 * w_scale)),
        "commands": args.pmc_commands or [],
    }
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    tag = args.workload if args.kv == "bf16" else f"{args.workload}_{args.kv}"
    out = os.path.join(ROOT, "profiles", f"traffic_{tag}.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="decode", choices=WORKLOADS)
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle CPU time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--timing-steps", type=int, default=200,
                    help="steps of the event-timed pass (at most --steps)")
    ap.add_argument("--replicas", type=int, default=0, help="input replicas (0 = >= 1 GiB total)")
    ap.add_argument("--graph-layers", type=int, default=0,
                    help="also time L layers' calls eagerly and as one captured HIP graph")
    ap.add_argument("--kv", default="bf16", choices=("bf16", "fp8"),
                    help="K/V pool format: bf16, or OCP FP8 E4M3 with per-KV-head scales (rpa_forward_fp8)")
    ap.add_argument("--append", action="store_true",
                    help="each step also writes its new K/V rows into the pages (rpa_forward_append)")
    ap.add_argument("--configs", default="all",
                    help="other workloads timed in the same run and reported under `configs`: "
                         "'all' (default), a comma-separated list, or '' for none")
    ap.add_argument("--stack", action="store_true",
                    help="also time one step of a 5 window-1024 : 1 global layer stack, eagerly and as "
                         "one captured HIP graph")
    ap.add_argument("--table", action="store_true",
                    help="run one call per entry of the planner's tuning table and print its kernels' times")
    ap.add_argument("--decode-max-rows", type=int, default=0,
                    help="with --table: RPA_OPT_DECODE_MAX_ROWS for every call (0: the library's table), to time "
                         "the choices the table does not make")
    ap.add_argument("--set", action="append", metavar="NAME=VALUE",
                    help="library option RPA_OPT_<NAME> for every call of the run (repeatable), "
                         "e.g. --set CONCURRENT=0 or --set FP8_STAGE=0")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run the elementwise calibration kernel (for counter runs)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs (no GPU needed)")
    ap.add_argument("--pmc-kernel", default="rpa_decode_kernel")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="markdown kernel statistics of a rocprofv3 --kernel-trace run (no GPU needed)")
    ap.add_argument("--pmc-commands", nargs="*")
    args = ap.parse_args(argv)

    if args.pmc_summary:
        return pmc_summary(args)
    if args.trace_summary:
        return trace_summary(args)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(how it would shard is described in the design notes); run with --gpus 1.",
              file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2
    return run(args)


if __name__ == "__main__":
    sys.exit(main())
