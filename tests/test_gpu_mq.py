"""Multi-query (speculative verify) decode: HIP path against the CPU oracle through the C ABI.

Each sequence carries M query tokens, its last M positions; query i attends to keys
0 .. len - M + i.  Tolerance as for single-token decode: |gpu - oracle| <= 2e-3 + 2e-3 |oracle|.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import decode_attention_04_amd as gd
from tests import workloads as W
from tests.gpu_util import DeviceCase, compare, dev_bf16, dev_i32, oracle_out, require_gpu

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a).view(np.uint32)


# the drafted block of the pages' speculative decoder is 7 tokens
VERIFY = [(7, 16, 8), (7, 4, 2), (4, 16, 4), (2, 24, 4), (16, 8, 8), (3, 8, 2)]   # (M, Hq, Hkv)


@pytest.mark.parametrize("D", [32, 64, 128, 256])
@pytest.mark.parametrize("M,Hq,Hkv", VERIFY)
def test_mq_matrix(D, M, Hq, Hkv):
    """Ragged lengths (including len < M, len = M and len = 0) and a NaN tail, several splits."""
    lens = [0, max(M - 1, 0), M, M + 1, 61, 517]
    say(f"[mq] D={D} M={M} Hq={Hq} Hkv={Hkv}")
    case = W.mq_case(len(lens), M, Hq, Hkv, D, 600, seq_lens=lens, seed=100 + D + M + Hq,
                     tail="nan")
    dc = DeviceCase(case)
    ref = oracle_out(case)
    for splits in (0, 1, 3, 40):
        compare(dc.run_host(splits), ref, f"mq D={D} M={M} Hq={Hq} Hkv={Hkv} splits={splits}")


def test_mq_verify_workload_bit_exact():
    """A verification step: 4 sequences of 4096 keys, 7 drafted tokens, GQA-2 hd128."""
    case = W.mq_case(4, 7, 16, 8, 128, 4096, seed=101)
    dc = DeviceCase(case)
    outs = [dc.run_host() for _ in range(3)]
    stats = compare(outs[0], oracle_out(case), "verify 4x7")
    say(f"[mq] verify workload: {stats}")
    for o in outs[1:]:
        assert np.array_equal(_bits(o), _bits(outs[0]))


def test_mq_one_query_is_single_token_decode():
    """M = 1 through gqa_decode_mq gives gqa_decode's bits."""
    case = W.mq_case(3, 1, 24, 4, 256, 1500, seq_lens=[1500, 700, 3], seed=102, scale=1 / 16)
    q = dev_bf16(case.q)
    k, v, lens = dev_bf16(case.k), dev_bf16(case.v), dev_i32(case.seq_lens)
    for splits in (0, 5):
        a = gd.gqa_decode_mq(q, k, v, lens, case.scale, num_splits=splits)
        b = gd.gqa_decode(q[:, 0].contiguous(), k, v, lens, case.scale, num_splits=splits)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(a[:, 0].cpu().numpy()), _bits(b.cpu().numpy()))


def test_mq_rows_match_single_token_calls():
    """Row i of a multi-query call equals gqa_decode of query i over its causal prefix, within
    tolerance (the splits of the two calls differ)."""
    case = W.mq_case(2, 5, 8, 4, 128, 300, seq_lens=[300, 40], seed=103)
    got = DeviceCase(case).run_host()
    k, v = dev_bf16(case.k), dev_bf16(case.v)
    for i in range(case.M):
        lens = dev_i32(case.seq_lens - case.M + i + 1)
        one = gd.gqa_decode(dev_bf16(np.ascontiguousarray(case.q[:, i])), k, v, lens, case.scale)
        torch.cuda.synchronize()
        compare(got[:, i], one.cpu().numpy().astype(np.float64), f"row {i}", atol=1e-5, rtol=1e-5)


@pytest.mark.parametrize("ps", [16, 32, 64])
def test_mq_paged(ps):
    case = W.mq_paged_case(4, 7, 16, 8, 128, ps, 400, [1000, 7, 3, 777], max_len=1024,
                           seed=104 + ps)
    dc = DeviceCase(case)
    ref = oracle_out(case)
    for splits in (0, 1, 9):
        compare(dc.run_host(splits), ref, f"mq paged ps={ps} splits={splits}")


def test_mq_even_shares(tune):
    case = W.mq_case(5, 4, 16, 4, 128, 2000, seq_lens=[2000, 4, 0, 999, 1500], seed=105)
    dc = DeviceCase(case)
    ref = oracle_out(case)
    for shares in ("1", "7", "64", "1000"):
        for fold in (1, 2):
            tune(shares=int(shares), fold=fold, partition=2)
            compare(dc.run_host(), ref, f"mq even shares={shares} fold={fold}")


def test_mq_rejects_too_many_rows():
    """M * G must fit the 16 MFMA columns (the binding's workspace query already refuses)."""
    case = W.mq_case(1, 5, 8, 2, 64, 64, seed=106)   # M * G = 20
    with pytest.raises(gd.GqaError):
        DeviceCase(case).run_host()
