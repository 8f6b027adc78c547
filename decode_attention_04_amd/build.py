"""Compile the HIP library (gfx950 only) in-tree: decode_attention_04_amd/libgqa_decode.so."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "gqa_decode.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgqa_decode.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the kernels' leading scalar arguments are preloaded into SGPRs at launch
    "-mllvm", "-amdgpu-kernarg-preload-count=10",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build(out: str = LIB, extra: list[str] | None = None, verbose: bool = False) -> str:
    """Always recompiles; writes atomically (each process through its own temporary file)."""
    tmp = f"{out}.{os.getpid()}.tmp"
    cmd = [HIPCC, *FLAGS, *(extra or []), "-I", INCLUDE, SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
