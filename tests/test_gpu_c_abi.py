"""The C ABI from a plain C program (tests/c_abi/gqa_c_caller.c, built by the package build):
hipMalloc'd buffers, gqa_decode / gqa_paged_decode / gqa_decode_noalloc, gqa_decode_partials +
gqa_decode_combine, gqa_decode_fp8 and gqa_decode_mq on ragged cases, checked against the CPU
oracle elementwise (|gpu - oracle| <= 2e-3 + 2e-3 |oracle|)."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

from tests.c_abi import build as c_caller
from tests.gpu_util import require_gpu

pytestmark = pytest.mark.gpu


def test_c_caller_on_the_gpu():
    require_gpu()
    exe = c_caller.OUT
    assert os.path.exists(exe), f"{exe} is not built; run __graft_entry__.build()"
    print("[c abi] running the C caller", flush=True)
    sys.stdout.flush()
    res = subprocess.run([exe, "gpu"], capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr, flush=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "gpu checks: ok" in res.stdout
