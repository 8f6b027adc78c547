"""The C ABI from a plain C program (tests/c_abi/gqa_c_caller.c: no Python, no torch), host
checks only: argument rejections, plans, the tuning, status strings.  Needs no GPU."""
from __future__ import annotations

import subprocess

from tests.c_abi import build as c_caller


def test_c_caller_host_checks(tmp_path):
    exe = c_caller.build(str(tmp_path / "gqa_c_caller"))
    res = subprocess.run([exe, "host"], capture_output=True, text=True, timeout=60)
    print(res.stdout, res.stderr)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "host checks: ok" in res.stdout
