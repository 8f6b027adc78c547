"""Seeded random shapes through every entry point: HIP path against the CPU oracle.

Each case draws the cache kind (contiguous / paged, bf16 / E4M3, one or several query tokens),
head_dim, group size, kv heads, batch, ragged lengths (zeros included), page size, the split
count, for some cases the even partition with a share count, and where the partials are folded (by the plan's
default, in a combine kernel, or in the split kernel itself), so that the plan's branches (fixed or
even partition, one-tile or key-range workgroups, direct or combined, packed or plain PV columns,
one launch or two) are crossed with each other rather than one at a time.  Tolerance as everywhere:
|gpu - oracle| <= 2e-3 + 2e-3 |oracle|, and a second call gives the same bits.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

from tests import workloads as W
from tests.gpu_util import DeviceCase, compare, oracle_out, require_gpu

pytestmark = pytest.mark.gpu

N_CASES = 120


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def draw(i: int) -> dict:
    """The i-th random case (a pure function of i)."""
    rng = np.random.default_rng(7000 + i)
    kind = ["contig", "paged", "fp8", "fp8_paged", "mq", "mq_paged"][i % 6]
    fp8 = kind.startswith("fp8")
    D = int(rng.choice([64, 128, 256] if fp8 else [32, 64, 128, 256]))
    M = int(rng.integers(2, 8)) if kind.startswith("mq") else 1
    groups = [g for g in (1, 2, 3, 4, 6, 8, 16) if M * g <= 16]
    G = int(rng.choice(groups))
    Hkv = int(rng.choice([1, 2, 4]))
    B = int(rng.integers(1, 7))
    S_max = int(rng.integers(1, 1300))
    lens = rng.integers(0, S_max, size=B, endpoint=True)
    lens[rng.random(B) < 0.2] = 0
    if M > 1:
        lens = np.maximum(lens, 0)
    splits = int(rng.choice([0, 0, 1, int(rng.integers(2, 60))]))
    shares = str(int(rng.choice([0, 1, 5, 64, 300]))) if rng.random() < 0.4 else None
    page_size = int(rng.choice([16, 32, 64, 128, 48]))
    fold = (i // 6) % 3  # 0: the plan's default, 1: combine kernel, 2: in the split kernel
    return dict(kind=kind, D=D, M=M, G=G, Hkv=Hkv, B=B, S_max=S_max, lens=[int(x) for x in lens],
                splits=splits, shares=shares, page_size=page_size, fold=fold, seed=9000 + i)


def build(c: dict) -> W.Case:
    Hq = c["G"] * c["Hkv"]
    B, D, lens, seed = c["B"], c["D"], c["lens"], c["seed"]
    kind = c["kind"]
    if kind in ("contig", "fp8", "mq"):
        S_max = max(c["S_max"], 1)
        if kind == "contig":
            return W.contig_case(B, Hq, c["Hkv"], D, S_max, seq_lens=lens, seed=seed, tail="nan")
        if kind == "fp8":
            return W.fp8_contig_case(B, Hq, c["Hkv"], D, S_max, seq_lens=lens, seed=seed)
        return W.mq_case(B, c["M"], Hq, c["Hkv"], D, S_max, seq_lens=lens, seed=seed, tail="nan")
    ps = c["page_size"]
    max_len = max(max(lens), 1)
    pages = sum((n + ps - 1) // ps for n in lens) + 3
    if kind == "paged":
        return W.paged_case(B, Hq, c["Hkv"], D, ps, pages, seq_lens=lens, max_len=max_len, seed=seed)
    if kind == "fp8_paged":
        return W.fp8_paged_case(B, Hq, c["Hkv"], D, ps, pages, seq_lens=lens, max_len=max_len, seed=seed)
    return W.mq_paged_case(B, c["M"], Hq, c["Hkv"], D, ps, pages, lens, max_len=max_len, seed=seed)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(tune, i):
    c = draw(i)
    say(f"[random] {i}: {c}")
    # a case that names a share count asks for the even partition (small jobs plan fixed splits)
    tune(shares=int(c["shares"] or 0), fold=c["fold"], partition=2 if c["shares"] is not None else 0)
    case = build(c)
    dc = DeviceCase(case)
    got = dc.run_host(c["splits"])
    compare(got, oracle_out(case), f"random case {i} {c}")
    again = dc.run_host(c["splits"])
    assert np.array_equal(np.ascontiguousarray(got).view(np.uint32),
                          np.ascontiguousarray(again).view(np.uint32)), "not bit-exact across runs"
