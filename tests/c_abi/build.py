"""Compile the plain C caller of the library's C ABI (test infrastructure): gqa_c_caller.c,
linked against the built HIP library and the CPU oracle."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "gqa_c_caller.c")
OUT = os.path.join(HERE, "gqa_c_caller")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(out: str = OUT) -> str:
    """Always recompiles (gcc, C11 with GNU extensions); writes atomically.  The libraries are
    found at run time next to the source tree ($ORIGIN-relative for the in-tree binary, and by
    absolute path)."""
    lib_dir = os.path.join(ROOT, "decode_attention_04_amd")
    oracle_dir = os.path.join(ROOT, "oracle")
    rpath = ":".join(["$ORIGIN/../../decode_attention_04_amd", "$ORIGIN/../../oracle", lib_dir, oracle_dir,
                      os.path.join(ROCM, "lib")])
    tmp = f"{out}.{os.getpid()}.tmp"
    cmd = ["gcc", "-std=gnu11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC, "-o", tmp,
           "-L", lib_dir, "-lgqa_decode", "-L", oracle_dir, "-loracle", "-L", os.path.join(ROCM, "lib"),
           "-lamdhip64", "-lm", f"-Wl,-rpath,{rpath}"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed ({res.returncode}):\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
