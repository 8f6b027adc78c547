"""Benchmark: GQA flash-decode µs/call and achieved HBM GB/s on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one gqa_decode (or gqa_paged_decode) call: the split kernel and the
combine, over one batch of synthetic seeded inputs already resident in HBM.
The K timed calls are captured once into a HIP graph and replayed, so the
host's per-call launch cost (Python + ctypes + hipLaunchKernel) does not
throttle the GPU; the eager per-call time is reported beside it.
Consecutive steps cycle through R copies of the inputs (more than 1 GiB in
total, several times the 256 MB Infinity Cache) so each call reads its K/V
from HBM, not from cache.  Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attention µs/call + achieved HBM GB/s (% of peak), GQA-6 hd256 ctx 4096"
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--splits", type=int, default=0, help="0 = the library's heuristic")
    ap.add_argument("--rotate-bytes", type=float, default=2.0 * 2**30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import decode_attention_04_amd as gd
    from tests import workloads as W
    from tests.gpu_util import DeviceCase

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    gd.load()
    name = args.workload or W.HEADLINE
    case = W.make(name)
    base = DeviceCase(case)
    algo_bytes = case.algorithmic_bytes()
    kv_bytes = case.k.nbytes + case.v.nbytes
    R = max(1, min(256, math.ceil(args.rotate_bytes / kv_bytes)))
    sets = [base] + [None] * (R - 1)
    for i in range(1, R):
        d = object.__new__(DeviceCase)
        d.case = case
        d.q, d.k, d.v = base.q.clone(), base.k.clone(), base.v.clone()
        d.seq_lens = base.seq_lens.clone()
        d.page_table = None if base.page_table is None else base.page_table.clone()
        sets[i] = d
    cap = case.capacity
    plan = gd.gqa_decode_plan(case.B, case.Hq, case.Hkv, case.D, cap, case.page_size,
                              args.splits, torch.cuda.get_device_properties(0).multi_processor_count)
    need = gd.gqa_decode_workspace_bytes(case.B, case.Hq, case.Hkv, case.D, cap, case.page_size,
                                         args.splits)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
    outs = [torch.empty((case.B, case.Hq, case.D), dtype=torch.float32, device="cuda")
            for _ in range(R)]
    def step(i, stream):
        sets[i % R].run(args.splits, out=outs[i % R], workspace=ws, stream=stream)

    # eager calls: W untimed warm-up steps, then a short timed eager run (reported, not the value)
    cur = torch.cuda.current_stream()
    for i in range(args.warmup):
        step(i, cur)
    torch.cuda.synchronize()
    n_eager = min(args.steps, 500)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(cur)
    for i in range(n_eager):
        step(i, cur)
    e1.record(cur)
    torch.cuda.synchronize()
    eager_us = e0.elapsed_time(e1) * 1e3 / n_eager

    # the timed region: exactly K calls, captured once into a HIP graph and replayed, so the
    # host's per-call launch cost does not throttle the GPU
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        step(0, side)
    cur.wait_stream(side)
    with torch.cuda.graph(graph):
        gs = torch.cuda.current_stream()
        for i in range(args.steps):
            step(i, gs)
    graph.replay()  # graph warm-up (not timed)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(cur)
    graph.replay()
    ev1.record(cur)
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / args.steps
    us = ms_per_step * 1e3
    gbs = algo_bytes / (ms_per_step * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = oracle.max_threads()
        t0 = time.perf_counter()
        calls = 0
        while True:
            if case.paged:
                oracle.paged_decode(case.q, case.k, case.v, case.seq_lens, case.page_table,
                                    case.scale)
            else:
                oracle.decode(case.q, case.k, case.v, case.seq_lens, case.scale)
            calls += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or el / calls * (calls + 1) > 3 * args.cpu_seconds:
                break
        cpu = {"value": round(algo_bytes * calls / el / 1e9, 4), "unit": "GB/s",
               "us_per_call": round(el / calls * 1e6, 1), "cores": threads, "kind": "oracle",
               "sample": f"{calls} full calls of {name} through the fp64 C oracle "
                         f"({el:.1f} s, {threads} OpenMP threads)"}

    line = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_call": round(us, 3),
        "eager_us_per_call": round(eager_us, 3),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 q/K/V)",
        "config": {"workload": name, "batch": case.B, "q_heads": case.Hq, "kv_heads": case.Hkv,
                   "head_dim": case.D, "capacity": cap, "page_size": case.page_size,
                   "sum_len": int(case.seq_lens.sum()), "algorithmic_bytes": algo_bytes,
                   "plan": plan.as_dict(), "rotated_sets": R, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "timed": "whole call (split kernel + combine), graph-replayed, event-timed"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
