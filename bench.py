"""Benchmark: GQA flash-decode µs/call and achieved HBM GB/s on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one gqa_decode (or gqa_paged_decode) call: the split kernel and the
combine, over one batch of synthetic seeded inputs already resident in HBM.
The K timed calls are captured once into a HIP graph and replayed at least 5
times; the value is the median replay (min and max beside it), so the host's
per-call launch cost (Python + ctypes + hipLaunchKernel) does not throttle the
GPU; the eager per-call time is reported beside it.  Consecutive steps cycle
through R copies of the inputs (more than 1 GiB in total, several times the
256 MB Infinity Cache) so each call reads its K/V from HBM, not from cache; the
same calls on one input set are reported apart as the cache-warm figure.  The
split and combine kernels are timed alone the same way.  Prints ONE JSON line
(with --all, one per workload).
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
    ap.add_argument("--all", action="store_true",
                    help="one line per workload (all five), instead of the headline workload only")
    ap.add_argument("--reps", type=int, default=5,
                    help="replays of the K-call graph that are timed (at least 5; median reported)")
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
    ap.add_argument("--summarize-counters", nargs="+", metavar="PMC_DIR",
                    help="print a markdown table of the per-dispatch averages of every counter in "
                         "these rocprofv3 --pmc output directories, per kernel of this library")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="per-kernel durations from a rocprofv3 --kernel-trace output directory of a "
                         "bench.py run with the same --steps/--reps: all dispatches, and the timed "
                         "replays of the one-kernel graphs (each kernel's last steps*reps dispatches)")
    ap.add_argument("--no-warm", action="store_true",
                    help="skip the cache-warm figure (one input set), e.g. under a counter run")
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


def combine_read_bytes(case, plan, piece_cost=4):
    """Bytes the combine kernel reads (the partials of every piece) and writes (the output).
    Fixed splits: every (sequence, kv head) has num_splits pieces.  Even shares: the pieces of
    each segment are the shares holding a tile of it (the library's share arithmetic, mirrored
    here for the byte count only)."""
    import numpy as np
    G = case.M * case.Hq // case.Hkv
    per_piece = G * (case.D + 2) * 4
    out_bytes = case.B * case.M * case.Hq * case.D * 4
    if plan.direct:
        return 0, 0
    if plan.partition == 0:
        return case.B * case.Hkv * plan.num_splits * per_piece, out_bytes
    tt = plan.tile_tokens
    lens = np.minimum(np.maximum(case.seq_lens.astype(np.int64), 0), case.capacity)
    tiles = (lens + tt - 1) // tt
    span = np.where(tiles > 0, tiles + piece_cost, 0)
    N = int(span.sum()) * case.Hkv
    P = plan.grid
    segs = int((tiles > 0).sum()) * case.Hkv
    long_ok = (not case.paged) and case.kv == "bf16"
    if long_ok and segs > 0 and N >= (128 + piece_cost) * segs:
        P = (P + 1) // 2   # one share per CU for long contiguous segments
    share_of = lambda x: ((x + 1) * P + N - 1) // N - 1
    begin = lambda w: w * N // P
    pieces, z = 0, 0
    for b in range(case.B):
        for _ in range(case.Hkv):
            n = int(tiles[b])
            if n:
                w0, w1 = share_of(z), share_of(z + n - 1)
                pieces += sum(1 for w in range(w0, w1 + 1) if begin(w) < begin(w + 1))
            z += int(span[b])
    return pieces * per_piece, out_bytes


def stats(samples):
    """median, min, max of per-call times (ms)."""
    v = sorted(samples)
    return v[len(v) // 2], v[0], v[-1]


def measure(name, args, with_cpu):
    """One workload: its JSON line (see the module docstring)."""
    import numpy as np
    import torch

    import decode_attention_04_amd as gd
    from tests import workloads as W
    from tests.gpu_util import DeviceCase

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
    outs = [torch.empty(oshape, dtype=torch.float32, device="cuda") for _ in range(R)]
    rot = [R]   # input sets the calls cycle through (1 for the cache-warm figure)

    def full(i, stream):
        sets[i % rot[0]].run(args.splits, out=outs[i % rot[0]], workspace=ws, stream=stream)

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

    def graph_time(fn, k, reps):
        """ms per call of `fn` for each of `reps` replays of one HIP graph of k calls (after one
        untimed replay), timed with HIP events on the stream the graph is replayed on."""
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
        out = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(cur)
            graph.replay()
            e1.record(cur)
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) / k)
        return out

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

    # The timed region: replays of one HIP graph of exactly K whole calls (the host's per-call
    # launch cost does not throttle the GPU); the value is the median replay.
    reps = max(5, args.reps)
    full_ms = graph_time(full, args.steps, reps)
    ms_per_step, full_min, full_max = stats(full_ms)
    gbs = algo_bytes / (ms_per_step * 1e-3) / 1e9
    # The split kernel alone (the dominant kernel) and the combine alone, each replayed the same
    # way, on the stream they are launched on.
    one_kernel = plan.direct or plan.fused   # a call is the split kernel alone
    if case.M == 1 and not one_kernel:
        split_ms = stats(graph_time(split_only, args.steps, reps))
        combine_ms = stats(graph_time(combine_only, args.steps, reps))
    else:   # one kernel per call (or multi-query calls, which have no split-only entry point)
        split_ms, combine_ms = (ms_per_step, full_min, full_max), (0.0,) * 3
    split_gbs = algo_bytes / (split_ms[0] * 1e-3) / 1e9
    # The same calls on ONE input set: K/V then sit in the 256 MB Infinity Cache when they fit
    # (reported apart, never as the value).
    warm_ms = (0.0,) * 3
    if not args.no_warm:
        rot[0] = 1
        warm_ms = stats(graph_time(full, args.steps, reps))
        rot[0] = R
    tuning = gd.gqa_decode_get_tuning().as_dict()
    cread, cwrite = combine_read_bytes(case, plan, tuning["piece_cost"])

    cpu = None
    if with_cpu:
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

    traffic = measured_traffic(name) if args.kv == "bf16" and case.M == 1 else None
    us3 = lambda t: round(t * 1e3, 3)
    return {
        "metric": METRIC if args.kv == "bf16" else METRIC + ", OCP FP8 E4M3 KV cache (1 B/element)",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_call": us3(ms_per_step),
        "us_per_call_min": us3(full_min),
        "us_per_call_max": us3(full_max),
        "replays": reps,
        "eager_us_per_call": round(eager_us, 3),
        "mall_warm_us_per_call": us3(warm_ms[0]) if not args.no_warm else None,
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
                   "plan": plan.as_dict(), "tuning": tuning, "rotated_sets": R,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "gqa_split_kernel", "achieved": round(split_gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(split_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel_us": us3(split_ms[0]), "kernel_us_min": us3(split_ms[1]),
                     "kernel_us_max": us3(split_ms[2]),
                     "timed": (f"split kernel alone: median of {reps} replays of a HIP graph of K "
                               "launches, HIP events on the launch stream")
                              if case.M == 1 and not one_kernel else
                              (f"whole calls, one kernel each (the split kernel "
                               f"{'writes the output directly' if plan.direct else 'folds its own partials'}): "
                               f"median of {reps} graph replays") if one_kernel else
                              f"whole multi-query calls: median of {reps} graph replays",
                     "combine": None if one_kernel else
                                {"kernel": "gqa_combine_narrow_kernel" if plan.max_pieces <= 16
                                 else "gqa_combine_kernel",
                                 "us": us3(combine_ms[0]), "us_min": us3(combine_ms[1]),
                                 "us_max": us3(combine_ms[2]),
                                 "bytes": cread + cwrite, "read_bytes": cread, "write_bytes": cwrite,
                                 "GB/s": round((cread + cwrite) / (combine_ms[0] * 1e-3) / 1e9, 2)
                                 if combine_ms[0] > 0 else None}},
        "cpu_baseline": cpu,
    }


KERNELS = ("gqa_split_kernel", "gqa_combine_narrow_kernel", "gqa_combine_kernel")


def summarize_counters(dirs):
    """Per-dispatch averages of each counter, per kernel: rows of one dispatch and counter are
    summed (rocprofv3 may report a counter per instance), then averaged over dispatches."""
    per = {}   # (kernel, counter) -> {dispatch: value}
    for d in dirs:
        for r in _counter_rows(d):
            name = r.get("Kernel_Name", "")
            kern = next((k for k in KERNELS if k in name), None)
            if kern is None:
                continue
            key = (kern, r["Counter_Name"])
            disp = (d, r["Dispatch_Id"])
            per.setdefault(key, {})
            per[key][disp] = per[key].get(disp, 0.0) + float(r["Counter_Value"])
    counters = sorted({c for _, c in per})
    kernels = [k for k in KERNELS if any((k, c) in per for c in counters)]
    print("| counter | " + " | ".join(kernels) + " |")
    print("|---|" + "---|" * len(kernels))
    for c in counters:
        cells = []
        for k in kernels:
            v = per.get((k, c))
            cells.append(f"{sum(v.values()) / len(v):,.0f} ({len(v)})" if v else "")
        print(f"| {c} | " + " | ".join(cells) + " |")


def summarize_trace(directory, timed):
    """Durations (ns) of this library's kernels in a kernel-trace CSV: every dispatch, and the
    last `timed` dispatches of each (the timed replays of its one-kernel graph in bench.py)."""
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as f:
            rows.extend(csv.DictReader(f))
    print("| kernel | dispatches | mean ns (all) | timed replays: n | mean ns | median ns | min | max |")
    print("|---|---|---|---|---|---|---|---|")
    for k in KERNELS:
        d = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
                   for r in rows if k in r.get("Kernel_Name", "") and
                   not any(o != k and o in r.get("Kernel_Name", "") and len(o) > len(k) for o in KERNELS))
        if not d:
            continue
        allv = [x for _, x in d]
        last = sorted(allv[-timed:])
        print(f"| {k} | {len(allv)} | {sum(allv) / len(allv):,.0f} | {len(last)} | "
              f"{sum(last) / len(last):,.0f} | {last[len(last) // 2]:,} | {last[0]:,} | {last[-1]:,} |")


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.steps * max(5, args.reps))
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.summarize_pmc:
        from tests import workloads as W
        summarize_pmc(*args.summarize_pmc, args.workload or W.HEADLINE)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)
    import torch

    import decode_attention_04_amd as gd
    from tests import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    gd.load()
    names = list(W.WORKLOADS) if args.all else [args.workload or W.HEADLINE]
    for name in names:
        line = measure(name, args, with_cpu=not args.no_cpu_baseline)
        print(json.dumps(line), flush=True)
        torch.cuda.empty_cache()
    if args.copy_calibration:
        copy_calibration()


if __name__ == "__main__":
    main()
