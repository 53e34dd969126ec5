#!/usr/bin/env python3
"""Throughput of ragged paged attention on one MI355X.

    python bench.py [--workload decode] [--steps K] [--warmup W] [--gpus 1]

A step is one ``rpa_forward`` call over one batch of seeded synthetic input
(bf16 N(0,1) Q/K/V, shuffled page tables) already resident in HBM.  The
default workload is the decode batch: 128 single-token sequences with kv_len
~ U[64, 640], 8 query heads sharing one KV head of width 256, 128-token pages.

So that no step finds its inputs in the 256 MB last-level cache, the bench
keeps R replicas of the inputs (at least 1 GiB in total) and step i reads
replica i mod R.  Per-step HIP events on the launch stream give the kernel
time behind ``roofline.achieved``; the wall clock over the K timed steps gives
``value`` and ``ms_per_step``.  The oracle's CPU time on a bounded sample of
the same workload is reported as ``cpu_baseline``.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention tokens/s + achieved TFLOP/s (prefill) and KV GB/s (decode), % of peak"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
LLC_BYTES = 256 << 20
KERNEL_SOURCE = os.path.join(ROOT, "ragged_paged_attention_forward_amd", "csrc", "rpa_kernels.hip")

# workload -> (dominant kernel name prefix, roofline bound)
DOMINANT = {
    "decode": ("rpa_decode_kernel", "hbm"),
    "tiny": ("rpa_prefill_kernel", "mfma"),
    "swa_prefill": ("rpa_prefill_kernel", "mfma"),
    "global_prefill": ("rpa_prefill_kernel", "mfma"),
    "mixed": ("rpa_prefill_kernel", "mfma"),
    "mixed_swa": ("rpa_prefill_kernel", "hbm"),
}


def kernel_source_hash() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if still current."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, budget_s: float):
    """Time the fp64 oracle on a bounded sample of the workload on the host cores."""
    import torch
    import oracle.rpa_oracle as ora
    import rpa_workloads as wl
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    cores = min(len(os.sched_getaffinity(0)), max(1, blas_threads))
    inp = wl.make_inputs(w)
    cu = inp.cu_q_lens.tolist()
    t_total = cu[-1]
    # sample: whole sequences for short ones; a strided set of rows for long prefills
    rng = np.random.default_rng(w.seed)
    order = rng.permutation(w.num_seqs)
    done_tokens = 0
    t0 = time.perf_counter()
    rows_per_call = 64
    desc = []
    for s in order:
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
        desc.append(len(rows))
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": done_tokens / el, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done_tokens} of {t_total} query tokens ({len(desc)} sequences, up to "
                      f"{rows_per_call} rows each) in {el:.1f} s, fp64 numpy",
            "seconds": round(el, 2)}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode", choices=sorted(DOMINANT))
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle CPU time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--replicas", type=int, default=0, help="input replicas (0 = >= 1 GiB total)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(sharding is described in the design notes); run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import rpa_workloads as wl
    from ragged_paged_attention_forward_amd import RaggedPagedAttention, metrics

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    w = wl.by_name(args.workload)
    host = wl.make_inputs(w)
    seqs = w.seqs
    t_q = w.total_q
    per_replica = sum(t.numel() * t.element_size() for t in (host.q, host.k_pages, host.v_pages)) * 2
    reps = args.replicas or max(2, int(np.ceil(4 * LLC_BYTES / per_replica)))
    replicas = []
    for _ in range(reps):
        d = host.to(dev)
        replicas.append((d, torch.empty_like(d.q)))
    cu = host.cu_q_lens.numpy()
    kv = host.kv_lens.numpy()

    attn = RaggedPagedAttention(w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size,
                                w.num_seqs, w.max_pages_per_seq, t_q)
    info, _ = attn.plan(cu, kv, w.window)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        d, out = replicas[i % reps]
        attn.forward(d.q, d.k_pages, d.v_pages, d.page_table, cu, kv, w.window, w.scale, out=out,
                     stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step(args.warmup + i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])

    ms_per_step = wall * 1e3 / args.steps
    kernel_ms = float(np.mean(ev_ms))
    flops = metrics.flops(seqs, w.window, w.num_q_heads, w.head_dim)
    alg_bytes = metrics.total_bytes(seqs, w.window, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                    w.page_size)
    kvb = metrics.kv_bytes(seqs, w.window, w.num_kv_heads, w.head_dim)
    assert info["visible_pairs"] == metrics.visible_pairs(seqs, w.window)

    kname, bound = DOMINANT[args.workload]
    if bound == "hbm":
        achieved = alg_bytes / (kernel_ms * 1e-3) / 1e9
        peak, unit = HBM_PEAK_GBS, "GB/s"
    else:
        achieved = flops / (kernel_ms * 1e-3) / 1e12
        peak, unit = MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    roofline = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": load_traffic(args.workload),
                "kernel": kname, "kernel_ms_mean": round(kernel_ms, 5),
                "kernel_ms_p10": round(float(np.percentile(ev_ms, 10)), 5),
                "kernel_ms_p90": round(float(np.percentile(ev_ms, 90)), 5),
                "algorithmic_bytes": int(alg_bytes), "algorithmic_flops": int(flops)}

    res = {
        "metric": METRIC,
        "value": round(t_q * args.steps / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "description": w.description, "seed": w.seed,
                   "num_seqs": w.num_seqs, "q_tokens": t_q, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "page_size": w.page_size, "window": w.window, "replicas": reps,
                   "parallelism": "single GPU"},
        "tflops": round(flops / (kernel_ms * 1e-3) / 1e12, 3),
        "kv_gbps": round(kvb / (kernel_ms * 1e-3) / 1e9, 1),
        "plan": info,
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(res), flush=True)
    attn.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
