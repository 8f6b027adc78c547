"""gqa_decode_noalloc (the library's static per-GPU scratch instead of a workspace) against
gqa_decode through the C ABI (needs an MI355X).

Same plan, same kernels: the outputs must be identical bit for bit, on two calls in a row with the
second one smaller (the shared scratch keeps the first call's partials, which the second must not
read), under both fold modes (the in-kernel fold's counters live in the scratch too), and a call
needing more scratch than the array holds is refused before any launch.
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

SCRATCH_BYTES = 4 << 20


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def noalloc(dc: DeviceCase, splits: int = 0) -> np.ndarray:
    c = dc.case
    out = torch.full((c.B, c.Hq, c.D), float("nan"), dtype=torch.float32, device="cuda")
    gd.gqa_decode_noalloc(dc.q, dc.k, dc.v, dc.seq_lens, c.scale, out, num_splits=splits)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("fold", [1, 2], ids=["kernel", "fused"])
def test_noalloc_matches_gqa_decode_two_calls(tune, fold):
    """A large call, then a smaller one: each equals gqa_decode's output bit for bit and the
    oracle within tolerance."""
    tune(fold=fold)
    first = W.make("gqa6_d256_ctx4096")
    second = W.contig_case(2, 16, 2, 128, 3000, seq_lens=[3000, 1234], seed=120, tail="nan")
    for case, splits in ((first, 0), (second, 0), (second, 7)):
        say(f"[noalloc] {case.name} fold={fold} splits={splits}")
        need = gd.gqa_decode_workspace_bytes(case.B, case.Hq, case.Hkv, case.D, case.capacity, 0, splits)
        assert 0 < need <= SCRATCH_BYTES
        dc = DeviceCase(case)
        got = noalloc(dc, splits)
        ref = dc.run_host(splits)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
        compare(got, oracle_out(case), f"noalloc {case.name} splits={splits}")


def test_noalloc_batched_even_shares():
    """Even shares (a batch of ragged sequences, one of them empty) through the static scratch."""
    case = W.contig_case(8, 32, 4, 128, 4096, seq_lens=[4096, 1, 0, 2048, 3000, 17, 4000, 999], seed=121)
    dc = DeviceCase(case)
    got = noalloc(dc)
    assert np.array_equal(got.view(np.uint32), dc.run_host().view(np.uint32))
    compare(got, oracle_out(case), "noalloc batched")
    assert np.all(got[2] == 0)


def test_noalloc_refuses_more_than_its_scratch():
    """A plan needing more than 4 MiB of scratch returns GQA_ERR_TOO_LARGE and writes nothing."""
    B, Hq, Hkv, D, S = 16, 64, 8, 256, 4096   # 16 fixed splits: 16.8 MB of partials
    need = gd.gqa_decode_workspace_bytes(B, Hq, Hkv, D, S, 0, 16)
    assert need > SCRATCH_BYTES
    q = torch.zeros((B, Hq, D), dtype=torch.int16, device="cuda")
    k = torch.zeros((B, Hkv, S, D), dtype=torch.int16, device="cuda")   # real buffers of full size
    v = torch.zeros((B, Hkv, S, D), dtype=torch.int16, device="cuda")
    lens = torch.full((B,), S, dtype=torch.int32, device="cuda")
    out = torch.full((B, Hq, D), 7.0, dtype=torch.float32, device="cuda")
    lib = gd.load()
    rc = lib.gqa_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), lens.data_ptr(), B, Hq, Hkv, D, S,
                                0.1, out.data_ptr(), 16, None)
    assert rc == 7 and gd.STATUS_NAMES[rc] == "GQA_ERR_TOO_LARGE"
    torch.cuda.synchronize()
    assert bool((out == 7.0).all().item())
