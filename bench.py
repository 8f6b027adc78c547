"""Benchmark: GQA flash-decode µs/call and achieved HBM GB/s on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME | --all]
                    [--ab FIELD=VALUE[,...]]

A step is one gqa_decode (or gqa_paged_decode) call: the split kernel and the
combine, over one batch of synthetic seeded inputs already resident in HBM.
The K timed calls are captured once into a HIP graph, so the host's per-call
launch cost (Python + ctypes + hipLaunchKernel) does not throttle the GPU; the
eager per-call time is reported beside it.  Consecutive steps cycle through R
copies of the inputs (more than 1 GiB in total, several times the 256 MB
Infinity Cache) so each call reads its K/V from HBM, not from cache; the same
calls on one input set are reported apart as the cache-warm figure.  The split
and combine kernels are captured alone the same way.  All graphs (with --all,
those of all five workloads) are then replayed in at least 5 rounds, each round
replaying every graph once in a fixed order (A B C A B C ...); the value is the
median round (min and max beside it).  Prints ONE JSON line (with --all, one per
workload).  --ab FIELD=VALUE compares a tuning variant with the current tuning
the same way (A B A B ...), one line per workload.
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
    ap.add_argument("--ab", metavar="FIELD=VALUE[,...]",
                    help="A/B mode: whole calls under the current tuning (A) against the tuning "
                         "with these gqa_tuning_t fields replaced (B), replayed alternately; one "
                         "line per workload (e.g. --ab fold=2 or --ab qk_mode=1)")
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
    long_ok = (not case.paged) and case.kv == "bf16"
    if plan.partition == 2:   # proportional splits: ceil(n / L) pieces per segment
        P = plan.grid - case.B * case.Hkv
        N = int(tiles.sum()) * case.Hkv
        segs = int((tiles > 0).sum()) * case.Hkv
        if long_ok and segs > 0 and N >= 128 * segs:
            P = (P + 1) // 2
        L = max(1, -(-N // P)) if N > 0 else 1
        pieces = int(((tiles + L - 1) // L).sum()) * case.Hkv
        return pieces * per_piece, out_bytes
    span = np.where(tiles > 0, tiles + piece_cost, 0)
    N = int(span.sum()) * case.Hkv
    P = plan.grid
    segs = int((tiles > 0).sum()) * case.Hkv
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


def parse_ab(spec):
    """'fold=2,qk_mode=1' -> {'fold': 2, 'qk_mode': 1} (fields of gqa_tuning_t)."""
    out = {}
    for item in spec.split(","):
        key, _, val = item.partition("=")
        if not key or not val:
            raise SystemExit(f"--ab wants FIELD=VALUE[,FIELD=VALUE...], got {spec!r}")
        out[key.strip()] = int(val)
    return out


class SkipWorkload(Exception):
    """A workload this run's options do not apply to (e.g. M * G > 16 query rows per kv head)."""


class Workload:
    """One workload on the device: R rotated copies of its seeded inputs (R * KV bytes above
    --rotate-bytes, several times the 256 MB Infinity Cache), one output per copy, one workspace
    large enough for every tuning in `tunings`, and the three call forms that are timed: the whole
    call, the split kernel alone and the combine alone."""

    def __init__(self, name, args, tunings=({},)):
        import torch

        import decode_attention_04_amd as gd
        from tests import workloads as W
        from tests.gpu_util import DeviceCase

        self.name, self.args = name, args
        case = W.make(name, kv=args.kv)
        if args.queries > 1:
            if args.kv != "bf16":
                sys.exit("--queries > 1 runs on the bf16 cache")
            if args.queries * (case.Hq // case.Hkv) > 16:
                raise SkipWorkload(f"{name}: {args.queries} queries x G = {case.Hq // case.Hkv} "
                                   "exceeds the 16 query rows of one kv head; skipped")
            case = W.with_queries(case, args.queries)
        self.case = case
        base = DeviceCase(case)
        self.algo_bytes = case.algorithmic_bytes()
        kv_bytes = case.k.nbytes + case.v.nbytes
        self.R = max(1, min(256, math.ceil(args.rotate_bytes / kv_bytes)))
        self.sets = [base]
        for _ in range(1, self.R):
            d = object.__new__(DeviceCase)
            d.case = case
            d.q, d.k, d.v = base.q.clone(), base.k.clone(), base.v.clone()
            d.seq_lens = base.seq_lens.clone()
            d.page_table = None if base.page_table is None else base.page_table.clone()
            self.sets.append(d)
        need = 0
        for t in tunings:
            with gd.tuning(**t):
                need = max(need, gd.gqa_decode_workspace_bytes(case.B, case.M * case.Hq, case.Hkv,
                                                               case.D, case.capacity,
                                                               case.page_size, args.splits))
        self.ws = gd.new_workspace(max(need, gd.COUNTER_BYTES))
        oshape = (case.B, case.Hq, case.D) if case.M == 1 else (case.B, case.M, case.Hq, case.D)
        self.outs = [torch.empty(oshape, dtype=torch.float32, device="cuda") for _ in range(self.R)]
        self.rot = self.R   # input sets the calls cycle through (1 for the cache-warm figure)

    def plan(self):
        """The library's plan for this workload under the current tuning."""
        import torch

        import decode_attention_04_amd as gd
        c = self.case
        plan_fn = gd.gqa_decode_plan_fp8 if c.kv == "fp8" else gd.gqa_decode_plan
        return plan_fn(c.B, c.M * c.Hq, c.Hkv, c.D, c.capacity, c.page_size, self.args.splits,
                       torch.cuda.get_device_properties(0).multi_processor_count)

    def full(self, i, stream):
        j = i % self.rot
        self.sets[j].run(self.args.splits, out=self.outs[j], workspace=self.ws, stream=stream)

    def split_only(self, i, stream):
        import decode_attention_04_amd as gd
        c, d, o, n = self.case, self.sets[i % self.R], self.outs[i % self.R], self.args.splits
        if c.kv == "fp8":
            if c.paged:
                gd.gqa_paged_decode_fp8_partials(d.q, d.k, d.v, d.seq_lens, d.page_table, c.scale,
                                                 c.k_scale, c.v_scale, out=o, workspace=self.ws,
                                                 num_splits=n, stream=stream)
            else:
                gd.gqa_decode_fp8_partials(d.q, d.k, d.v, d.seq_lens, c.scale, c.k_scale,
                                           c.v_scale, out=o, workspace=self.ws, num_splits=n,
                                           stream=stream)
        elif c.paged:
            gd.gqa_paged_decode_partials(d.q, d.k, d.v, d.seq_lens, d.page_table, c.scale, out=o,
                                         workspace=self.ws, num_splits=n, stream=stream)
        else:
            gd.gqa_decode_partials(d.q, d.k, d.v, d.seq_lens, c.scale, out=o, workspace=self.ws,
                                   num_splits=n, stream=stream)

    def combine_only(self, i, stream):
        import decode_attention_04_amd as gd
        c = self.case
        fn = gd.gqa_decode_combine_fp8 if c.kv == "fp8" else gd.gqa_decode_combine
        fn(self.ws, self.sets[i % self.R].seq_lens, self.outs[i % self.R], c.B, c.Hq, c.Hkv, c.D,
           c.capacity, c.page_size, self.args.splits, stream=stream)

    def warm_up(self):
        """W untimed calls, then a short eager run: µs per call with the host's launch path in
        the loop (reported beside the value, never as it)."""
        import torch
        cur = torch.cuda.current_stream()
        for i in range(self.args.warmup):
            self.full(i, cur)
        torch.cuda.synchronize()
        n = min(self.args.steps, 500)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(cur)
        for i in range(n):
            self.full(i, cur)
        e1.record(cur)
        torch.cuda.synchronize()
        self.eager_us = e0.elapsed_time(e1) * 1e3 / n


def capture(fn, k):
    """One HIP graph of k calls of `fn` (after one eager call on a side stream), replayed once
    untimed."""
    import torch
    cur = torch.cuda.current_stream()
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
    return graph


def replay_rounds(graphs, k, reps):
    """ms per call of every graph in `graphs` (a list of (key, graph)), `reps` rounds: each round
    replays every graph once in the listed order (A B C A B C ...), each replay bracketed by HIP
    events on the stream it is replayed on.  Returns {key: [ms per call, one per round]}."""
    import torch
    cur = torch.cuda.current_stream()
    out = {key: [] for key, _ in graphs}
    for _ in range(reps):
        for key, g in graphs:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(cur)
            g.replay()
            e1.record(cur)
            torch.cuda.synchronize()
            out[key].append(e0.elapsed_time(e1) / k)
    return out


def timed_graphs(w, args):
    """The graphs timed for a workload's line: the whole call; the split kernel and the combine
    alone (two-kernel plans of one-query calls); the whole call over one input set (cache-warm)."""
    plan = w.plan()
    w.one_kernel = bool(plan.direct or plan.fused)   # a call is the split kernel alone
    w.plan_now = plan
    g = [((w.name, "full"), capture(w.full, args.steps))]
    if w.case.M == 1 and not w.one_kernel:
        g.append(((w.name, "split"), capture(w.split_only, args.steps)))
        g.append(((w.name, "combine"), capture(w.combine_only, args.steps)))
    if not args.no_warm:
        w.rot = 1
        g.append(((w.name, "warm"), capture(w.full, args.steps)))
        w.rot = w.R
    return g


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, args):
    """The fp64 oracle on this host's cores (all OpenMP threads) over full calls of the same
    workload for about --cpu-seconds, then one thread for a few calls (context only)."""
    import oracle
    case = w.case

    def call():
        if case.M > 1 and case.paged:
            oracle.paged_decode_mq(case.q, case.k, case.v, case.seq_lens, case.page_table, case.scale)
        elif case.M > 1:
            oracle.decode_mq(case.q, case.k, case.v, case.seq_lens, case.scale)
        elif case.kv == "fp8" and case.paged:
            oracle.paged_decode_fp8(case.q, case.k, case.v, case.seq_lens, case.page_table,
                                    case.scale, case.k_scale, case.v_scale)
        elif case.kv == "fp8":
            oracle.decode_fp8(case.q, case.k, case.v, case.seq_lens, case.scale, case.k_scale,
                              case.v_scale)
        elif case.paged:
            oracle.paged_decode(case.q, case.k, case.v, case.seq_lens, case.page_table, case.scale)
        else:
            oracle.decode(case.q, case.k, case.v, case.seq_lens, case.scale)

    def timed(budget):
        t0 = time.perf_counter()
        calls = 0
        while True:
            call()
            calls += 1
            el = time.perf_counter() - t0
            if el >= budget or el / calls * (calls + 1) > 3 * budget:
                return calls, el

    threads = oracle.max_threads()
    calls, el = timed(args.cpu_seconds)
    oracle.set_threads(1)
    try:
        calls1, el1 = timed(args.cpu_seconds / 4)
    finally:
        oracle.set_threads(threads)
    return {"value": round(w.algo_bytes * calls / el / 1e9, 4), "unit": "GB/s",
            "us_per_call": round(el / calls * 1e6, 1), "cores": threads, "kind": "oracle",
            "sample": f"{calls} full calls of {w.name} through the fp64 C oracle "
                      f"({el:.1f} s, {threads} OpenMP threads)",
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "one_thread_us_per_call": round(el1 / calls1 * 1e6, 1), "one_thread_calls": calls1}


def line_for(w, times, args, reps, with_cpu):
    """The JSON line of one workload from its timed rounds."""
    import decode_attention_04_amd as gd
    case, plan = w.case, w.plan_now
    ms_per_step, full_min, full_max = stats(times[(w.name, "full")])
    gbs = w.algo_bytes / (ms_per_step * 1e-3) / 1e9
    if (w.name, "split") in times:
        split_ms = stats(times[(w.name, "split")])
        combine_ms = stats(times[(w.name, "combine")])
    else:   # one kernel per call (or multi-query calls, which have no split-only entry point)
        split_ms, combine_ms = (ms_per_step, full_min, full_max), (0.0,) * 3
    split_gbs = w.algo_bytes / (split_ms[0] * 1e-3) / 1e9
    warm = times.get((w.name, "warm"))
    tuning = gd.gqa_decode_get_tuning().as_dict()
    cread, cwrite = combine_read_bytes(case, plan, tuning["piece_cost"])
    one_kernel = w.one_kernel
    traffic = measured_traffic(w.name) if args.kv == "bf16" and case.M == 1 else None
    us3 = lambda t: round(t * 1e3, 3)
    order = "replays in alternating order with the workload's other graphs" + \
        (" and the other workloads'" if args.all else "")
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
        "eager_us_per_call": round(w.eager_us, 3),
        "mall_warm_us_per_call": us3(stats(warm)[0]) if warm else None,
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if args.kv == "bf16" else "fp8-e4m3 KV, bf16 q and MFMA",
        "data": "synthetic (seeded N(0,1) bf16 q/K/V)" if args.kv == "bf16" else
                "synthetic (seeded N(0,1) bf16 q; K/V the same draws rounded to E4M3 at scale 1/16)",
        "config": {"workload": w.name, "batch": case.B, "queries_per_sequence": case.M,
                   "q_heads": case.Hq, "kv_heads": case.Hkv,
                   "head_dim": case.D, "capacity": case.capacity, "page_size": case.page_size,
                   "sum_len": int(case.seq_lens.sum()), "algorithmic_bytes": w.algo_bytes,
                   "plan": plan.as_dict(), "tuning": tuning, "rotated_sets": w.R,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "gqa_split_kernel", "achieved": round(split_gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(split_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel_us": us3(split_ms[0]), "kernel_us_min": us3(split_ms[1]),
                     "kernel_us_max": us3(split_ms[2]),
                     "timed": (f"split kernel alone: median of {reps} replays of a HIP graph of K "
                               f"launches ({order}), HIP events on the launch stream")
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
        "cpu_baseline": cpu_baseline(w, args) if with_cpu else None,
    }


def run_lines(names, args):
    """The default and --all modes: every workload's graphs captured first, then timed in rounds
    that alternate over all of them; one line per workload."""
    import torch
    reps = max(5, args.reps)
    loads, graphs = [], []
    for name in names:
        try:
            w = Workload(name, args)
        except SkipWorkload as e:
            if len(names) == 1:
                sys.exit(str(e))
            print(e, file=sys.stderr, flush=True)
            continue
        w.warm_up()
        graphs += timed_graphs(w, args)
        loads.append(w)
    times = replay_rounds(graphs, args.steps, reps)
    del graphs
    for w in loads:
        print(json.dumps(line_for(w, times, args, reps, with_cpu=not args.no_cpu_baseline)), flush=True)
    torch.cuda.synchronize()


def run_ab(names, args):
    """--ab: for each workload, whole calls under the current tuning (A) and under the tuning with
    the given fields replaced (B), each a HIP graph of K calls, replayed A B A B ... for --reps
    rounds; one line per workload with both medians."""
    import torch

    import decode_attention_04_amd as gd
    spec = parse_ab(args.ab)
    reps = max(5, args.reps)
    for name in names:
        try:
            w = Workload(name, args, tunings=({}, spec))
        except SkipWorkload as e:
            if len(names) == 1:
                sys.exit(str(e))
            print(e, file=sys.stderr, flush=True)
            continue
        w.warm_up()
        base = gd.gqa_decode_get_tuning().as_dict()
        plan_a = w.plan()
        g_a = capture(w.full, args.steps)
        with gd.tuning(**spec):
            plan_b = w.plan()
            for i in range(args.warmup):
                w.full(i, torch.cuda.current_stream())
            g_b = capture(w.full, args.steps)
        times = replay_rounds([("a", g_a), ("b", g_b)], args.steps, reps)
        del g_a, g_b
        a, b = stats(times["a"]), stats(times["b"])
        side = lambda t, plan, ms: {"tuning": t, "plan": plan.as_dict(), "us_per_call": round(ms[0] * 1e3, 3),
                                     "us_per_call_min": round(ms[1] * 1e3, 3),
                                     "us_per_call_max": round(ms[2] * 1e3, 3),
                                     "GB/s": round(w.algo_bytes / (ms[0] * 1e-3) / 1e9, 2)}
        print(json.dumps({
            "mode": "ab", "workload": name, "kv": args.kv, "steps": args.steps, "replays": reps,
            "timed": f"whole calls: A and B graphs of K calls replayed alternately ({reps} rounds), "
                     "median, min and max per call",
            "a": side({k: base[k] for k in spec}, plan_a, a),
            "b": side(spec, plan_b, b),
            "b_over_a": round(b[0] / a[0], 4)}), flush=True)
        del w
        torch.cuda.empty_cache()


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


def summarize_trace(directory, steps, reps):
    """Durations (ns) of this library's kernels in a kernel-trace CSV of a bench.py run with the
    same --steps/--reps: every dispatch, and the timed replays of each kernel's one-kernel graph.
    Those replays are the runs of exactly `steps` consecutive dispatches of one kernel (a whole-call
    graph alternates split and combine; the untimed replay of a graph follows its capture-time
    call, so its run is longer); the last `reps` such runs are taken.  Where the split kernel is
    the whole call (direct or folded plans) its dispatches form one run, and the last
    steps * reps dispatches are the timed ones (a run with --no-warm)."""
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as f:
            rows.extend(csv.DictReader(f))

    def family(name):
        hits = [k for k in KERNELS if k in name]
        return max(hits, key=len) if hits else None

    seq = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"]),
                  family(r.get("Kernel_Name", ""))) for r in rows)
    seq = [(t, d, k) for t, d, k in seq if k is not None]
    runs = []   # (kernel, [durations]) of consecutive dispatches of one kernel
    for _, d, k in seq:
        if runs and runs[-1][0] == k:
            runs[-1][1].append(d)
        else:
            runs.append((k, [d]))
    print("| kernel | dispatches | mean ns (all) | timed replays: n | mean ns | median ns | min | max |")
    print("|---|---|---|---|---|---|---|---|")
    for k in KERNELS:
        allv = [d for _, d, kk in seq if kk == k]
        if not allv:
            continue
        exact = [v for kk, v in runs if kk == k and len(v) == steps]
        if exact:
            last = sorted(x for v in exact[-reps:] for x in v)
        else:
            last = sorted(allv[-steps * reps:])
        print(f"| {k} | {len(allv)} | {sum(allv) / len(allv):,.0f} | {len(last)} | "
              f"{sum(last) / len(last):,.0f} | {last[len(last) // 2]:,} | {last[0]:,} | {last[-1]:,} |")


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.steps, max(5, args.reps))
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.summarize_pmc:
        from tests import workloads as W
        summarize_pmc(*args.summarize_pmc, args.workload or W.HEADLINE)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)
    import torch

    import decode_attention_04_amd as gd
    from tests import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    gd.load()
    names = list(W.WORKLOADS) if args.all else [args.workload or W.HEADLINE]
    if args.ab:
        run_ab(names, args)
    else:
        run_lines(names, args)
    if args.copy_calibration:
        copy_calibration()


if __name__ == "__main__":
    main()
