"""Calls captured in a HIP graph (torch.cuda.graph) and replayed: every replay gives the bits of
the same call made eagerly, with eager library calls on the same workspace, other device work
and synchronisations between the replays (the calls enqueue only, never allocate when given
`out` and a workspace, and leave the arrival counters zero, so a replay needs no reset).

Plans covered: fixed splits with the combine kernel, even shares, the small in-kernel fold, a
paged cache, an E4M3 cache, multi-query rows, and the allocation-free entry point."""
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


CASES = {
    "fixed": lambda: W.contig_case(1, 24, 4, 256, 4096, seq_lens=[4000], seed=120, scale=1 / 16),
    "even": lambda: W.contig_case(12, 32, 4, 128, 3000, seq_lens=[3000, 17, 2500, 0, 999, 3000, 1, 2048,
                                                                  640, 2999, 1500, 33], seed=121),
    "fused_small": lambda: W.contig_case(1, 8, 2, 64, 512, seed=122),
    "paged": lambda: W.paged_case(6, 16, 4, 128, 32, 400, seq_lens=[1, 700, 2048, 31, 1200, 999],
                                  max_len=2048, seed=123),
    "fp8": lambda: W.fp8_contig_case(3, 16, 4, 128, 2000, seq_lens=[2000, 5, 1111], seed=124),
    "mq": lambda: W.mq_case(2, 3, 16, 4, 128, 1500, seq_lens=[1500, 40], seed=125),
    "noalloc": lambda: W.contig_case(2, 16, 2, 128, 3000, seq_lens=[3000, 1234], seed=126),
}


def _call(kind, dc, out, ws):
    if kind == "noalloc":
        c = dc.case
        gd.gqa_decode_noalloc(dc.q, dc.k, dc.v, dc.seq_lens, c.scale, out)
    else:
        dc.run(0, out=out, workspace=ws)


@pytest.mark.parametrize("kind", list(CASES))
def test_graph_replays_match_eager(kind):
    say(f"[graph] {kind}")
    case = CASES[kind]()
    dc = DeviceCase(case)
    c = case
    oshape = (c.B, c.Hq, c.D) if c.M == 1 else (c.B, c.M, c.Hq, c.D)
    other = W.contig_case(3, 8, 2, 128, 900, seq_lens=[900, 0, 450], seed=127)  # called between replays
    need = max(gd.gqa_decode_workspace_bytes(c.B, c.M * c.Hq, c.Hkv, c.D, c.capacity, c.page_size, 0),
               gd.gqa_decode_workspace_bytes(other.B, other.Hq, other.Hkv, other.D, other.capacity, 0, 0))
    ws = gd.new_workspace(max(need, gd.COUNTER_BYTES))
    ref_out = torch.empty(oshape, dtype=torch.float32, device="cuda")
    _call(kind, dc, ref_out, ws)
    torch.cuda.synchronize()
    eager = ref_out.cpu().numpy()
    compare(eager, oracle_out(case), f"graph {kind}: eager call")

    out = torch.empty(oshape, dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _call(kind, dc, out, ws)  # the eager call before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(kind, dc, out, ws)
    dother = DeviceCase(other)
    ref_other = oracle_out(other)
    junk = torch.randn(1 << 20, device="cuda")
    for r in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), eager.view(np.uint32)), f"{kind}: replay {r} differs"
        # eager work between replays: another plan on the same workspace, and other kernels
        o2 = dother.run(0, workspace=ws)
        junk.mul_(0.5).add_(1.0)
        torch.cuda.synchronize()
        compare(o2.cpu().numpy(), ref_other, f"graph {kind}: eager call between replays")
    del g
    torch.cuda.synchronize()
