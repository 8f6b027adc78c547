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


def measured_traffic(workload):
    """HBM bytes per split-kernel launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    src = os.path.join(ROOT, "decode_attention_04_amd", "csrc", "gqa_decode.hip")
    try:
        with open(path) as f:
            rec = json.load(f)
        with open(src, "rb") as f:
            digest = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != digest:
        return None
    w = rec.get("workloads", {}).get(workload)
    return None if w is None else w.get("hbm_bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--splits", type=int, default=0, help="0 = the library's heuristic")
    ap.add_argument("--queries", type=int, default=1,
                    help="query tokens per sequence (multi-query decode, gqa_decode_mq); "
                         "M * G must be <= 16")
    ap.add_argument("--kv", choices=("bf16", "fp8"), default="bf16",
                    help="cache element type: bf16 (the headline), or the workload's OCP FP8 E4M3 "
                         "form with per-tensor scales (gqa_decode_fp8)")
    ap.add_argument("--rotate-bytes", type=float, default=2.0 * 2**30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the benchmark, copy a 256 MiB buffer 5 times (a plain copy "
                         "kernel of known size, to scale rocprofv3 byte counters)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc output directories (FETCH_SIZE, WRITE_SIZE) "
                         "of a --copy-calibration run into profiles/traffic.json")
    return ap.parse_args()


COPY_BYTES = 256 * 2**20


def copy_calibration():
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()


def _counter_rows(directory):
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            rows.extend(csv.DictReader(f))
    return rows


def _per_dispatch(rows, counter, match):
    vals = [float(r["Counter_Value"]) for r in rows
            if r.get("Counter_Name") == counter and match(r.get("Kernel_Name", ""))]
    return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)


def summarize_pmc(fetch_dir, write_dir, workload):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the split kernel, scaled by what the
    same counters read for the plain copy kernel of COPY_BYTES, into profiles/traffic.json."""
    import hashlib
    fr, wr = _counter_rows(fetch_dir), _counter_rows(write_dir)
    is_split = lambda n: "gqa_split_kernel" in n
    f_split, nf = _per_dispatch(fr, "FETCH_SIZE", is_split)
    w_split, nw = _per_dispatch(wr, "WRITE_SIZE", is_split)

    # the calibration copies: the last five device-to-device copy dispatches of the run
    def calib(rows, counter):
        copies = [r for r in rows if "copyBuffer" in r.get("Kernel_Name", "")
                  and r.get("Counter_Name") == counter]
        copies.sort(key=lambda r: int(r["Dispatch_Id"]))
        vals = [float(r["Counter_Value"]) for r in copies[-5:]]
        return sum(vals) / len(vals) if vals else None
    f_copy, w_copy = calib(fr, "FETCH_SIZE"), calib(wr, "WRITE_SIZE")
    if None in (f_split, w_split, f_copy, w_copy):
        raise SystemExit("counter rows missing for the split or the copy kernel")
    f_scale = COPY_BYTES / (f_copy * 1024)   # true bytes per counted byte
    w_scale = COPY_BYTES / (w_copy * 1024)
    fetch_b = f_split * 1024 * f_scale
    write_b = w_split * 1024 * w_scale
    src = os.path.join(ROOT, "decode_attention_04_amd", "csrc", "gqa_decode.hip")
    with open(src, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    if rec.get("kernel_source_sha256") != digest:
        rec = {"kernel_source_sha256": digest, "workloads": {}}
    rec["note"] = ("HBM bytes per gqa_split_kernel launch: rocprofv3 FETCH_SIZE and WRITE_SIZE "
                   "(KiB per dispatch, one counter run each) scaled by the same counters read for "
                   f"a plain {COPY_BYTES} B device-to-device copy kernel")
    rec["workloads"][workload] = {
        "fetch_kib_per_dispatch": round(f_split, 1), "write_kib_per_dispatch": round(w_split, 1),
        "copy_fetch_kib": round(f_copy, 1), "copy_write_kib": round(w_copy, 1),
        "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
        "dispatches": [nf, nw],
        "hbm_bytes_per_launch": int(round(fetch_b + write_b)),
        "fetch_bytes_per_launch": int(round(fetch_b)), "write_bytes_per_launch": int(round(write_b)),
    }
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    print(json.dumps(rec["workloads"][workload]))


def main():
    args = parse()
    if args.summarize_pmc:
        from tests import workloads as W
        summarize_pmc(*args.summarize_pmc, args.workload or W.HEADLINE)
        return
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
    case = W.make(name, kv=args.kv)
    if args.queries > 1:
        if args.kv != "bf16":
            sys.exit("--queries > 1 runs on the bf16 cache")
        case = W.with_queries(case, args.queries)
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
    plan_fn = gd.gqa_decode_plan_fp8 if case.kv == "fp8" else gd.gqa_decode_plan
    plan = plan_fn(case.B, case.M * case.Hq, case.Hkv, case.D, cap, case.page_size,
                   args.splits, torch.cuda.get_device_properties(0).multi_processor_count)
    need = gd.gqa_decode_workspace_bytes(case.B, case.M * case.Hq, case.Hkv, case.D, cap, case.page_size,
                                         args.splits)
    ws = gd.new_workspace(max(need, gd.COUNTER_BYTES))
    oshape = (case.B, case.Hq, case.D) if case.M == 1 else (case.B, case.M, case.Hq, case.D)
    outs = [torch.empty(oshape, dtype=torch.float32, device="cuda")
            for _ in range(R)]
    def full(i, stream):
        sets[i % R].run(args.splits, out=outs[i % R], workspace=ws, stream=stream)

    def split_only(i, stream):
        d = sets[i % R]
        if case.kv == "fp8":
            if case.paged:
                gd.gqa_paged_decode_fp8_partials(d.q, d.k, d.v, d.seq_lens, d.page_table,
                                                 case.scale, case.k_scale, case.v_scale,
                                                 out=outs[i % R], workspace=ws,
                                                 num_splits=args.splits, stream=stream)
            else:
                gd.gqa_decode_fp8_partials(d.q, d.k, d.v, d.seq_lens, case.scale, case.k_scale,
                                           case.v_scale, out=outs[i % R], workspace=ws,
                                           num_splits=args.splits, stream=stream)
        elif case.paged:
            gd.gqa_paged_decode_partials(d.q, d.k, d.v, d.seq_lens, d.page_table, case.scale,
                                         out=outs[i % R], workspace=ws, num_splits=args.splits,
                                         stream=stream)
        else:
            gd.gqa_decode_partials(d.q, d.k, d.v, d.seq_lens, case.scale, out=outs[i % R],
                                   workspace=ws, num_splits=args.splits, stream=stream)

    combine_fn = gd.gqa_decode_combine_fp8 if case.kv == "fp8" else gd.gqa_decode_combine

    def combine_only(i, stream):
        combine_fn(ws, sets[i % R].seq_lens, outs[i % R], case.B, case.Hq, case.Hkv,
                   case.D, cap, case.page_size, args.splits, stream=stream)

    cur = torch.cuda.current_stream()

    def graph_time(fn, k):
        """ms per call of `fn` over k calls captured in one HIP graph (one untimed replay first)."""
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            fn(0, side)
        cur.wait_stream(side)
        with torch.cuda.graph(graph):
            gs = torch.cuda.current_stream()
            for i in range(k):
                fn(i, gs)
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(cur)
        graph.replay()
        e1.record(cur)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / k

    # W untimed warm-up steps, then a short timed eager run (reported beside the value)
    for i in range(args.warmup):
        full(i, cur)
    torch.cuda.synchronize()
    n_eager = min(args.steps, 500)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(cur)
    for i in range(n_eager):
        full(i, cur)
    e1.record(cur)
    torch.cuda.synchronize()
    eager_us = e0.elapsed_time(e1) * 1e3 / n_eager

    # The timed region: exactly K whole calls, captured once into a HIP graph and replayed,
    # so the host's per-call launch cost does not throttle the GPU.
    ms_per_step = graph_time(full, args.steps)
    us = ms_per_step * 1e3
    gbs = algo_bytes / (ms_per_step * 1e-3) / 1e9
    # The dominant kernel alone (the split-KV partial kernel; K launches in one graph), and the
    # combine alone, each on the stream they are launched on.
    if case.M == 1:
        split_ms = graph_time(split_only, args.steps)
        combine_ms = graph_time(combine_only, args.steps) if not plan.direct else 0.0
    else:   # multi-query calls have no split-only entry point: the roofline uses whole calls
        split_ms, combine_ms = ms_per_step, 0.0
    split_gbs = algo_bytes / (split_ms * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = oracle.max_threads()
        t0 = time.perf_counter()
        calls = 0
        while True:
            if case.M > 1 and case.paged:
                oracle.paged_decode_mq(case.q, case.k, case.v, case.seq_lens, case.page_table,
                                       case.scale)
            elif case.M > 1:
                oracle.decode_mq(case.q, case.k, case.v, case.seq_lens, case.scale)
            elif case.kv == "fp8" and case.paged:
                oracle.paged_decode_fp8(case.q, case.k, case.v, case.seq_lens, case.page_table,
                                        case.scale, case.k_scale, case.v_scale)
            elif case.kv == "fp8":
                oracle.decode_fp8(case.q, case.k, case.v, case.seq_lens, case.scale, case.k_scale,
                                  case.v_scale)
            elif case.paged:
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

    traffic = measured_traffic(name) if args.kv == "bf16" else None
    line = {
        "metric": METRIC if args.kv == "bf16" else METRIC + ", OCP FP8 E4M3 KV cache (1 B/element)",
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
        "dtype": "bf16" if args.kv == "bf16" else "fp8-e4m3 KV, bf16 q and MFMA",
        "data": "synthetic (seeded N(0,1) bf16 q/K/V)" if args.kv == "bf16" else
                "synthetic (seeded N(0,1) bf16 q; K/V the same draws rounded to E4M3 at scale 1/16)",
        "config": {"workload": name, "batch": case.B, "queries_per_sequence": case.M,
                   "q_heads": case.Hq, "kv_heads": case.Hkv,
                   "head_dim": case.D, "capacity": cap, "page_size": case.page_size,
                   "sum_len": int(case.seq_lens.sum()), "algorithmic_bytes": algo_bytes,
                   "plan": plan.as_dict(), "rotated_sets": R, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "gqa_split_kernel", "achieved": round(split_gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(split_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel_us": round(split_ms * 1e3, 3),
                     "combine_us": round(combine_ms * 1e3, 3),
                     "timed": "K launches of the split kernel alone in one HIP graph, HIP events"
                              if case.M == 1 else "K whole multi-query calls in one HIP graph"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    if args.copy_calibration:
        copy_calibration()


if __name__ == "__main__":
    main()
