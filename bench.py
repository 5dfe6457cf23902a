#!/usr/bin/env python3
"""Benchmark of sparse MLA decode on one MI355X.

A step is one pass of the whole hot path over one batch: the host split
planner, the split-KV decode kernel and (for more than one split) the stage-2
merge kernel.  The default workload is the bf16 decode of T=8 tokens x 64
heads, 2048 top-k + 128 sliding-window indices (1% invalid) into a
32768-row pool.  Inputs are seeded synthetic data resident in HBM before the
timed region; the K timed steps are captured into one HIP graph and replayed
once, bracketed by device synchronisation.

The `roofline` object reports the decode kernel alone: algorithmic bytes per
launch over its average duration, measured with HIP events on the stream it
runs on (a graph of back-to-back decode launches).  `cpu_baseline` times the
float64 oracle on the host on a bounded sample of the same workload.

Prints one JSON line.  --gpus above 1 is refused: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "sparse-MLA decode µs/call + achieved HBM GB/s (% roofline), T x ctx matrix"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
BF16_MFMA_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=1, help="workload index 0..4 (1 = bf16 T=8 H=64 K=2176)")
    ap.add_argument("--cell", type=str, default=None, help="T x ctx matrix cell T:ctx:variant instead of --config")
    ap.add_argument("--splits", type=int, default=None, help="override the planner's split count")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--kernel-launches", type=int, default=50)
    return ap.parse_args()


def make_workload(args):
    import workloads as wl
    if args.cell:
        T, ctx, var = args.cell.split(":")
        return wl.matrix_cell(int(T), int(ctx), var)
    return wl.config(args.config)


def to_device(w, dev):
    import torch
    import sparse_mla_decode_index_amd as smd
    a = w.arrays

    def bf(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    if w.kv_dtype == "bf16":
        pool = smd.KVPool.bf16(bf(a["kv"]))
    else:
        pool = smd.KVPool.fp8(torch.from_numpy(a["nope"]).to(dev), torch.from_numpy(a["scale"]).to(dev),
                              bf(a["rope"]))
    return dict(q_nope=bf(a["q_nope"]), q_rope=bf(a["q_rope"]), pool=pool,
                indices=torch.from_numpy(a["indices"]).to(dev), sink=torch.from_numpy(a["sink"]).to(dev))


def cpu_baseline(w, target_s: float):
    """Time the float64 oracle on index rows of the same workload until about
    target_s seconds of CPU work; scale to a whole call."""
    from oracle import ref
    a = w.arrays
    pool = {"kv": a["kv"]} if w.kv_dtype == "bf16" else {"nope": a["nope"], "scale": a["scale"], "rope": a["rope"]}
    R = w.num_index_rows
    qps = w.q_per_seq
    done, t_used = 0, 0.0
    t0 = time.perf_counter()
    while t_used < target_s and done < 100000:
        b = done % R
        ref.sparse_mla_decode(a["q_nope"][b * qps:(b + 1) * qps], a["q_rope"][b * qps:(b + 1) * qps], pool,
                              a["indices"][b:b + 1], a["sink"], w.softmax_scale, qps)
        done += 1
        t_used = time.perf_counter() - t0
    per_row = t_used / done
    per_call = per_row * R
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = 1
    return per_call, done, t_used, cores


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)
    import torch
    import sparse_mla_decode_index_amd as smd
    import workloads as wl

    dev = torch.device("cuda:0")
    w = make_workload(args)
    d = to_device(w, dev)
    T, H, qps = w.num_tokens, w.num_heads, w.q_per_seq
    K = w.arrays["indices"].shape[1]
    kvd = smd.KV_BF16 if w.kv_dtype == "bf16" else smd.KV_FP8_E4M3_UE8M0
    R = w.num_index_rows

    def plan():
        return args.splits or smd.plan_num_kv_splits(R, H, K, qps, kvd)

    s = plan()
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    po = torch.empty((T, H, s, 512), dtype=torch.float32, device=dev)
    pl = torch.empty((T, H, s), dtype=torch.float32, device=dev)

    def step(num_splits):
        smd.sparse_mla_decode(d["q_nope"], d["q_rope"], d["pool"], d["indices"], d["sink"], w.softmax_scale,
                              num_splits=num_splits, q_per_seq=qps, out=out, lse=lse,
                              partial_o=po if num_splits > 1 else None, partial_lse=pl if num_splits > 1 else None)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step(plan())
    torch.cuda.synchronize()

    # K whole-path steps captured into one graph (planner runs on the host per step)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(args.steps):
            step(s)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        g.replay()  # one untimed replay of the captured graph
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for _ in range(args.steps):
        s_k = plan()
    assert s_k == s
    with torch.cuda.stream(stream):
        g.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # decode kernel alone: back-to-back launches in a graph, HIP events on its stream
    nk = args.kernel_launches
    gk = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gk, stream=stream):
        for _ in range(nk):
            if s > 1:
                smd.sparse_mla_decode(d["q_nope"], d["q_rope"], d["pool"], d["indices"], d["sink"],
                                      w.softmax_scale, num_splits=s, q_per_seq=qps, partials_only=True,
                                      partial_o=po, partial_lse=pl)
            else:
                step(1)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        gk.replay()
        e0.record(stream)
        gk.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    kern_us = e0.elapsed_time(e1) * 1e3 / nk

    alg_bytes = wl.algorithmic_bytes(w)
    alg_flops = wl.algorithmic_flops(w)
    us_per_call = ms_per_step * 1e3
    gbs = alg_bytes / (us_per_call * 1e3)
    kern_gbs = alg_bytes / (kern_us * 1e3)
    kern_tfs = alg_flops / (kern_us * 1e6)
    t_hbm = alg_bytes / (HBM_PEAK_GBS * 1e3)
    t_mfma = alg_flops / (BF16_MFMA_PEAK_TFS * 1e6)
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(kern_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(kern_gbs / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        roof = {"bound": "mfma", "achieved": round(kern_tfs, 1), "peak": BF16_MFMA_PEAK_TFS, "unit": "TFLOP/s",
                "frac": round(kern_tfs / BF16_MFMA_PEAK_TFS, 4), "traffic": None}
    roof.update({"kernel": "smd::decode_kernel", "kernel_us": round(kern_us, 3),
                 "alg_bytes_per_launch": alg_bytes, "alg_flops_per_launch": alg_flops})

    res = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_call": round(us_per_call, 3),
        "tokens_per_s": round(T / (us_per_call * 1e-6), 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.kv_dtype == "bf16" else "fp8-e4m3/ue8m0 in, bf16 mfma",
        "data": "synthetic",
        "config": {"workload": w.name, "num_tokens": T, "num_heads": H, "q_per_seq": qps, "topk": K,
                   "pool_rows": w.pool_rows, "kv_dtype": w.kv_dtype, "num_splits": s, "parallelism": "1 gpu"},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        per_call, rows, secs, cores = cpu_baseline(w, args.cpu_seconds)
        res["cpu_baseline"] = {"value": round(alg_bytes / (per_call * 1e9), 4), "unit": "GB/s", "cores": cores,
                               "kind": "oracle", "us_per_call": round(per_call * 1e6, 1),
                               "sample": f"{rows} index rows of the same workload ({secs:.1f} s), "
                                         f"scaled to one call of {R} rows"}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
