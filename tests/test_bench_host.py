"""Host logic of bench.py (CPU only): picking the timed replays out of a kernel trace, and the
--ab field list."""
from __future__ import annotations

import csv
import os

import pytest

import bench

SPLIT = "void gqa_split_kernel<256, 1, false, 1, false, 0, 2, 0, 0>(SplitArgs)"
TREE = "void gqa_combine_kernel<4, 0>(float const*, float const*)"


def _write_trace(tmp_path, seq):
    d = tmp_path / "trace" / "host"
    os.makedirs(d)
    with open(d / "x_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        t = 1000
        for name, dur in seq:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + dur})
            t += dur + 500
    return str(tmp_path / "trace")


def _rows(out):
    rows = {}
    for line in out.splitlines():
        cells = [c.strip() for c in line.strip("|").split("|")]
        if cells and cells[0] in bench.KERNELS:
            rows[cells[0]] = cells
    return rows


def test_trace_picks_the_one_kernel_graph_replays(tmp_path, capsys):
    """Whole-call graphs alternate split and combine dispatches; the split-only and combine-only
    graphs are runs of exactly K dispatches; their capture-time call makes the untimed replay's
    run K + 1 long.  Only the timed rounds' runs may be picked."""
    K, reps = 4, 5
    seq = [(SPLIT, 9000), (TREE, 9000)] * 3                      # warm-up and eager calls
    seq += [(SPLIT, 9000), (TREE, 9000)] * (K + 1)                # full graph: capture call + replay
    seq += [(SPLIT, 7000)] * (K + 1) + [(TREE, 7000)] * (K + 1)   # one-kernel graphs, untimed
    for r in range(reps):
        seq += [(SPLIT, 6000), (TREE, 3000)] * K                 # timed whole calls
        seq += [(SPLIT, 5000 + r)] * K                           # timed split-only replay
        seq += [(TREE, 2000 + r)] * K                            # timed combine-only replay
    bench.summarize_trace(_write_trace(tmp_path, seq), K, reps)
    rows = _rows(capsys.readouterr().out)
    split, tree = rows["gqa_split_kernel"], rows["gqa_combine_kernel"]
    assert int(split[3]) == K * reps and int(tree[3]) == K * reps
    assert split[6] == "5,000" and split[7] == "5,004"     # min, max of the split-only rounds
    assert tree[6] == "2,000" and tree[7] == "2,004"


def test_trace_one_kernel_plans_take_the_last_dispatches(tmp_path, capsys):
    K, reps = 3, 5
    seq = [(SPLIT, 9000)] * 10 + [(SPLIT, 4000 + i) for i in range(K * reps)]
    bench.summarize_trace(_write_trace(tmp_path, seq), K, reps)
    split = _rows(capsys.readouterr().out)["gqa_split_kernel"]
    assert int(split[3]) == K * reps and split[6] == "4,000" and split[7] == "4,014"


def test_parse_ab():
    assert bench.parse_ab("fold=2") == {"fold": 2}
    assert bench.parse_ab("fold=2, qk_mode=1") == {"fold": 2, "qk_mode": 1}
    with pytest.raises(SystemExit):
        bench.parse_ab("fold")
