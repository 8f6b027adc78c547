"""The in-kernel fold (one launch) against the oracle and against the combine kernel (needs an
MI355X).

The split workgroup that writes the last partial of a group -- all pieces of a (sequence, kv
head) segment in the even partition, a node of the fold tree over fixed splits -- learns it from
an arrival ticket and folds the group itself.  Checked here: the five workloads at full size under
both fold modes, fixed split counts through every tree shape (one node, two and three levels),
bitwise agreement with the combine kernel where both fold the same partials in the same order,
zero rows for empty sequences that no piece covers, and the arrival counters back at zero after
every call.  Tolerance as everywhere: |gpu - oracle| <= 2e-3 + 2e-3 |oracle|.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import decode_attention_04_amd as gd
from tests import workloads as W
from tests.gpu_util import DeviceCase, compare, oracle_out, require_gpu

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def counters_zero(ws: torch.Tensor) -> bool:
    torch.cuda.synchronize()
    return bool((ws[:gd.COUNTER_BYTES] == 0).all().item())


def run_with(dc: DeviceCase, ws: torch.Tensor, splits: int = 0) -> np.ndarray:
    out = dc.run(splits, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def workspace_for(case: W.Case, splits: int = 0) -> torch.Tensor:
    need = gd.gqa_decode_workspace_bytes(case.B, case.M * case.Hq, case.Hkv, case.D, case.capacity,
                                         case.page_size, splits)
    return gd.new_workspace(max(need, gd.COUNTER_BYTES))


_REF = {}


def reference(name: str, case: W.Case) -> np.ndarray:
    """The oracle's output for one full-size workload (kept for the next fold mode only)."""
    if name not in _REF:
        _REF.clear()
        say(f"[fold] {name}: oracle")
        _REF[name] = oracle_out(case)
    return _REF[name]


@pytest.mark.parametrize("name", list(W.WORKLOADS))
@pytest.mark.parametrize("fold", [1, 2], ids=["kernel", "fused"])
def test_workload_fold_modes(tune, name, fold):
    tune(fold=fold)
    say(f"[fold] {name} fold={fold}: generating")
    case = W.make(name)
    dc = DeviceCase(case)
    plan = gd.gqa_decode_plan(case.B, case.Hq, case.Hkv, case.D, case.capacity, case.page_size)
    say(f"[fold] {name} fold={fold}: plan {plan.as_dict()}")
    assert plan.fused == (fold == 2 and not plan.direct)
    ws = workspace_for(case)
    outs = [run_with(dc, ws) for _ in range(3)]
    stats = compare(outs[0], reference(name, case), f"{name} fold={fold}")
    say(f"[fold] {name} fold={fold}: {stats}")
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32)), "not bit-exact across runs"
    assert counters_zero(ws), "arrival counters not back at zero"


@pytest.mark.parametrize("splits", [2, 5, 16, 17, 40, 64, 100, 256, 500])
def test_fused_fixed_split_counts(tune, splits):
    """Fold trees of one node (up to 16 splits), two levels and three levels (500 requested
    splits of a 8k-key cache: fan-in 16, 512 / 16 / 2 / 1 nodes), ragged lengths with a NaN tail
    and an empty sequence."""
    tune(fold=2)
    say(f"[fold] fixed splits={splits}")
    case = W.contig_case(3, 24, 4, 256, 8192, seq_lens=[8192, 1500, 0], seed=80, scale=1 / 16,
                         tail="nan")
    dc = DeviceCase(case)
    plan = gd.gqa_decode_plan(case.B, case.Hq, case.Hkv, case.D, case.capacity, 0, splits)
    assert plan.fused == 1 and plan.partition == 0
    ws = workspace_for(case, splits)
    a = run_with(dc, ws, splits)
    b = run_with(dc, ws, splits)
    compare(a, oracle_out(case), f"fused fixed splits={splits}")
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.all(a[2] == 0)
    assert counters_zero(ws)
    if plan.num_splits <= 16:
        # one node over all splits: the arithmetic of the thread-per-column combine
        with gd.tuning(fold=1):
            c = run_with(dc, ws, splits)
        assert np.array_equal(a.view(np.uint32), c.view(np.uint32))


def _even_cases():
    lens70 = np.random.default_rng(81).integers(0, 2305, 70)
    return [
        lambda: W.contig_case(10, 16, 4, 128, 5000, seq_lens=[1, 0, 700, 3, 5000, 17, 0, 2048, 1, 33], seed=82, tail="nan"),
        lambda: W.paged_case(16, 32, 8, 128, 32, 4000, max_len=8192, seed=83),
        lambda: W.contig_case(70, 16, 2, 128, 2304, seq_lens=lens70, seed=84),
        lambda: W.mq_case(12, 3, 16, 4, 128, 3000, seq_lens=[3000, 2, 0, 999, 1500, 2500] * 2, seed=85),
        lambda: W.fp8_contig_case(18, 16, 2, 128, 3000, seq_lens=[3000, 1, 0, 1500, 77, 2999] * 3, seed=86),
        lambda: W.fp8_paged_case(10, 16, 4, 128, 32, 400, seq_lens=[2048, 1, 0, 777, 1500] * 2, max_len=2048, seed=87),
    ]


@pytest.mark.parametrize("i", range(6))
def test_fused_even_matches_combine_bitwise(tune, i):
    """Even shares: the split kernel folds each segment's pieces with the thread-per-column
    combine's arithmetic, in the same order, and writes a segment held by one share straight to
    `out` -- so one launch and two give the same bits (bf16, paged, many sequences, multi-query
    rows, E4M3)."""
    case = _even_cases()[i]()
    say(f"[fold] even bitwise {case.name}")
    dc = DeviceCase(case)
    tune(fold=2, partition=2)
    ws = workspace_for(case)
    plan_fn = gd.gqa_decode_plan_fp8 if case.kv == "fp8" else gd.gqa_decode_plan
    plan = plan_fn(case.B, case.M * case.Hq, case.Hkv, case.D, case.capacity, case.page_size)
    assert plan.partition == 1 and plan.fused == 1 and plan.max_pieces <= 16
    one = run_with(dc, ws)
    assert counters_zero(ws)
    tune(fold=1, partition=2)
    two = run_with(dc, ws)
    compare(one, oracle_out(case), f"fused even {case.name}")
    assert np.array_equal(one.view(np.uint32), two.view(np.uint32))


@pytest.mark.parametrize("fold", [1, 2], ids=["kernel", "fused"])
def test_empty_sequences_write_zero_rows(tune, fold):
    """No piece covers a sequence of length 0; its output rows are still written (zeros) over an
    output buffer that held NaN, also for sequences past the launched workgroups' count."""
    tune(fold=fold, shares=3, partition=2)
    lens = [0, 2000, 0, 0, 1500, 0, 33, 0]
    case = W.contig_case(len(lens), 16, 4, 128, 2048, seq_lens=lens, seed=88)
    dc = DeviceCase(case)
    ws = workspace_for(case)
    out = torch.full((case.B, case.Hq, case.D), float("nan"), dtype=torch.float32, device="cuda")
    dc.run(0, out=out, workspace=ws)
    got = out.cpu().numpy()
    compare(got, oracle_out(case), f"empty rows fold={fold}")
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(got[b] == 0)
    assert counters_zero(ws)


def test_counters_survive_mixed_calls(tune):
    """One workspace through a sequence of calls of different shapes, partitions and fold
    modes (fused fixed trees, fused even shares, partials + combine): every result matches the
    oracle and the counters end at zero."""
    tune(fold=2)
    a = W.contig_case(1, 8, 1, 128, 40000, seed=89)                            # 256 splits: 2 levels
    b = W.paged_case(8, 16, 4, 128, 32, 700, max_len=4096, seed=90)             # even shares
    c = W.contig_case(2, 24, 4, 256, 3000, seq_lens=[3000, 2999], seed=91, scale=1 / 16)
    refs = {x.name: oracle_out(x) for x in (a, b, c)}
    dcs = {x.name: DeviceCase(x) for x in (a, b, c)}
    ws = gd.new_workspace(64 << 20)
    for rep in range(3):
        for x, splits in ((a, 0), (b, 0), (c, 7), (a, 300), (c, 0)):
            compare(run_with(dcs[x.name], ws, splits), refs[x.name], f"rep {rep} {x.name} {splits}")
        # the two-kernel path on the same workspace in between
        out = torch.empty((c.B, c.Hq, c.D), dtype=torch.float32, device="cuda")
        d = dcs[c.name]
        gd.gqa_decode_partials(d.q, d.k, d.v, d.seq_lens, c.scale, out=out, workspace=ws,
                               num_splits=5)
        gd.gqa_decode_combine(ws, d.seq_lens, out, c.B, c.Hq, c.Hkv, c.D, c.capacity, 0, 5)
        torch.cuda.synchronize()
        compare(out.cpu().numpy(), refs[c.name], f"rep {rep} partials + combine")
    assert counters_zero(ws)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("shares", [195, 1000])
@pytest.mark.parametrize("fold", [1, 2], ids=["kernel", "fused"])
def test_more_shares_than_positions(tune, kv, shares, fold):
    """More shares than positions on the tile axis: some shares hold no tile and write no
    partial, and the fold (combine kernel or in-kernel) skips their slots, with a different
    segment in each lane of the combine's waves."""
    tune(shares=shares, fold=fold, partition=2)
    lens = [0, 0, 205, 0, 175]
    make = W.fp8_contig_case if kv == "fp8" else W.contig_case
    case = make(5, 8, 4, 64, 1240, seq_lens=lens, seed=9080)
    dc = DeviceCase(case)
    ws = workspace_for(case)
    a = run_with(dc, ws)
    compare(a, oracle_out(case), f"{kv} shares={shares} fold={fold}")
    assert np.array_equal(a.view(np.uint32), run_with(dc, ws).view(np.uint32))
    assert counters_zero(ws)
